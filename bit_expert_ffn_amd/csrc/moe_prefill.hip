// Prefill path (T > 8): placeholder layout until the matrix-core kernels land.
#include "moe_internal.h"

namespace moe {

LargeLayout large_layout(int T, int k, int E, int H, int FF, int FFs, int qtype) {
    (void)E; (void)qtype;
    LargeLayout L{};
    size_t off = 0;
    auto take = [&](size_t b) { size_t o = off; off = (off + b + 255) & ~(size_t)255; return o; };
    const size_t n = (size_t)T * k;
    L.ids = take(n * 4);
    L.w = take(n * 4);
    L.a = take(n * FF * 4);
    L.as = take((size_t)T * FFs * 4);
    L.ypair = take(n * H * 4);
    L.ys = take((size_t)T * H * 4);
    L.total = off;
    return L;
}

}  // namespace moe
