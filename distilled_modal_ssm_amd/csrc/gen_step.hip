// gen_step.hip -- the prepare step of the deferred decode state, on its own.
//
// The decode recurrence of the Laughing Hyena Distillery review (主要发现:
// O(d) state and time per generated token), y = q (D u + Re sum R x),
// x <- lambda x + u, is evaluated with the addition of u deferred to the next
// token: the stored state is s = x - u_prev.  Prepare,
//     x = s + u_prev;  rho = Re sum_n R_n x_n;  s <- lambda x,
// needs nothing from the coming token; the projected stack runs it inside the
// previous layer's in_proj launch (dense.hip, launch_layer_gate), where the
// weight stream leaves HBM bandwidth to spare, and the gate of the token is
// then y = q (D u + rho), u_prev <- u.  This kernel runs it alone: at the
// start of generation, for the first layer.
//
// One thread per unit (batch row, two adjacent channels of a head): d 16-byte
// state loads, all in flight, then the readout, d 16-byte stores.
#include "hm_internal.hpp"

namespace hm {
namespace {

constexpr int kThreads = 256;

template <int DD>
__global__ __launch_bounds__(kThreads) void prepare_kernel(PrepArgs p) {
    const int64_t units = p.B * (p.D / 2);
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < units; u += (int64_t)gridDim.x * kThreads)
        prepare_unit<DD>(p, u);
}

}  // namespace

bool prepare_supported(int64_t d) { return d == 8 || d == 16 || d == 32; }

hipError_t launch_prepare(const PrepArgs &p, hipStream_t stream) {
    const int64_t units = p.B * (p.D / 2);
    if (units == 0) return hipSuccess;
    int64_t grid = (units + kThreads - 1) / kThreads;
    if (grid > 65536) grid = 65536;
    switch (p.d) {
        case 8: prepare_kernel<8><<<dim3((unsigned)grid), kThreads, 0, stream>>>(p); break;
        case 16: prepare_kernel<16><<<dim3((unsigned)grid), kThreads, 0, stream>>>(p); break;
        case 32: prepare_kernel<32><<<dim3((unsigned)grid), kThreads, 0, stream>>>(p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hm
