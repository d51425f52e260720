// route.hip -- the router kernel: one 256-thread workgroup per token runs the
// sigmoid + score-correction-bias top-K selection of route.hpp (colibri PR #684,
// engine commit, Stable LatentMoE bullet; PR #676 summary: top-16 of 896) and
// writes the slot-order result.
#include "device.hpp"
#include "launch.hpp"
#include "route.hpp"

namespace k3moe {

namespace {

using namespace route_detail;

// One workgroup of 4 waves per token; the routing weights renormalize the
// selected raw sigmoids, summed in slot order in double.
template <int PL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int T, int E, int K,
                                                    double top_p, int32_t* __restrict__ idx,
                                                    float* __restrict__ w, int32_t* __restrict__ n_kept) {
    __shared__ RouteScratch rs;
    extern __shared__ double sig_e[];  // [E] double sigmoid of each expert's logit
    const int t = blockIdx.x;
    route_block<PL>(logits + (size_t)t * E, bias, E, K, top_p, rs, sig_e, idx + (size_t)t * K, w + (size_t)t * K,
                    n_kept != nullptr ? n_kept + t : nullptr);
}

template <int PL>
hipError_t launch_pl(const float* logits, const float* bias, int T, int E, int K, double top_p, int32_t* idx,
                     float* w, int32_t* n_kept, hipStream_t stream) {
    hipLaunchKernelGGL(route_kernel<PL>, dim3(T), dim3(256), (size_t)E * sizeof(double), stream, logits, bias, T, E,
                       K, top_p, idx, w, n_kept);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* logits, const float* bias, int T, int E, int K, double top_p, int32_t* idx,
                        float* w, int32_t* n_kept, hipStream_t stream) {
    const int per_lane = route_per_lane(E);  // candidates per lane in each of 4 waves
    if (per_lane <= 1) return launch_pl<1>(logits, bias, T, E, K, top_p, idx, w, n_kept, stream);
    if (per_lane <= 2) return launch_pl<2>(logits, bias, T, E, K, top_p, idx, w, n_kept, stream);
    if (per_lane <= 4) return launch_pl<4>(logits, bias, T, E, K, top_p, idx, w, n_kept, stream);
    if (per_lane <= 8) return launch_pl<8>(logits, bias, T, E, K, top_p, idx, w, n_kept, stream);
    return launch_pl<16>(logits, bias, T, E, K, top_p, idx, w, n_kept, stream);
}

}  // namespace k3moe
