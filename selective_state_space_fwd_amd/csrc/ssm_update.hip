// ssm_update.hip -- single-token state update (decode) for gfx950.
//
// The persistent per-channel state of the ufo.work article "Mamba
// hardware-aware operator fusion and selective-scan parallelisation", §4.1:
// one token advances it in place by h_new = exp(dt A) h_old + dt B u (or the
// zero-order-hold term (exp(dt A) - 1) / A B u), and the output is
// y = (C . h_new + D u) silu(z).
//
// The step is a pure stream over the state (read + write of N floats per
// channel), so the mapping is chosen for coalescing: P lanes per channel,
// P = next power of two >= ceil(N / 4), each lane owning 4 consecutive states
// (one 16-byte access); consecutive lanes touch consecutive 16-byte pieces of
// the state, and the channel's partial dot products meet through a butterfly
// of P lanes.
#include "ssm_common.h"
#include "ssm_launch.h"

namespace ssm {

template <class IO, bool VEC>
__global__ __launch_bounds__(256) void update_kernel(UpdateArgs a, int P, int log2P) {
    using IT = typename IO::T;
    const IT *__restrict__ u = static_cast<const IT *>(a.u);
    const IT *__restrict__ dl = static_cast<const IT *>(a.delta);
    const IT *__restrict__ z = static_cast<const IT *>(a.z);
    const IT *__restrict__ Bm = static_cast<const IT *>(a.B);
    const IT *__restrict__ Cm = static_cast<const IT *>(a.C);
    IT *__restrict__ y = static_cast<IT *>(a.y);

    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t ch = gid >> log2P;                   // b * D + d
    const int l = static_cast<int>(gid & (P - 1));
    const bool ok = ch < a.Bsz * a.D;                  // whole P-lane groups agree
    const int64_t chs = ok ? ch : 0;
    const int64_t b = chs / a.D, d = chs % a.D;
    const int n0 = 4 * l;

    float acc = 0.0f;
    float uu = 0.0f;
    if (ok && n0 < a.N) {
        uu = IO::load(u, chs);
        const float dt = IO::load(dl, chs);
        const float w = dt * uu;
        float *st = a.state + chs * a.N + n0;
        const float *Ar = a.A + d * a.N + n0;
        const size_t bo = static_cast<size_t>(b) * a.N + n0;
        if (VEC) {
            float4 s = *reinterpret_cast<const float4 *>(st);
            const float4 A4 = *reinterpret_cast<const float4 *>(Ar);
            float sv[4] = {s.x, s.y, s.z, s.w};
            const float av[4] = {A4.x, A4.y, A4.z, A4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float xa = dt * (av[i] * kLog2e);
                const float dA = exp2_hw(xa);
                const float wi = a.zoh ? w * zoh_phi(xa * kLn2, dA) : w;
                sv[i] = __builtin_fmaf(dA, sv[i], wi * IO::load(Bm, bo + i));
                acc = __builtin_fmaf(IO::load(Cm, bo + i), sv[i], acc);
            }
            *reinterpret_cast<float4 *>(st) = make_float4(sv[0], sv[1], sv[2], sv[3]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (n0 + i < a.N) {
                    const float xa = dt * (Ar[i] * kLog2e);
                    const float dA = exp2_hw(xa);
                    const float wi = a.zoh ? w * zoh_phi(xa * kLn2, dA) : w;
                    const float sv = __builtin_fmaf(dA, st[i], wi * IO::load(Bm, bo + i));
                    st[i] = sv;
                    acc = __builtin_fmaf(IO::load(Cm, bo + i), sv, acc);
                }
            }
        }
    }
    // Sum over the P lanes of the channel (butterfly; fixed order per lane).
    for (int off = P >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (ok && l == 0) {
        if (a.Dskip) acc = __builtin_fmaf(a.Dskip[d], uu, acc);
        if (a.z) acc *= silu_f32(IO::load(z, chs));
        IO::store(y, chs, acc);
    }
}

template <class IO>
static hipError_t launch_update_io(const UpdateArgs &a, hipStream_t s) {
    const int groups = static_cast<int>((a.N + 3) / 4);
    int P = 1, log2P = 0;
    while (P < groups) { P <<= 1; ++log2P; }
    const int64_t threads = a.Bsz * a.D * P;
    const unsigned blocks = static_cast<unsigned>((threads + 255) / 256);
    const bool vec = (a.N % 4 == 0) &&
                     (reinterpret_cast<uintptr_t>(a.state) % 16 == 0) &&
                     (reinterpret_cast<uintptr_t>(a.A) % 16 == 0);
    if (vec)
        hipLaunchKernelGGL((update_kernel<IO, true>), dim3(blocks), dim3(256), 0, s, a, P, log2P);
    else
        hipLaunchKernelGGL((update_kernel<IO, false>), dim3(blocks), dim3(256), 0, s, a, P, log2P);
    return hipGetLastError();
}

hipError_t launch_update(const UpdateArgs &a, hipStream_t s) {
    return a.bf16 ? launch_update_io<BF16>(a, s) : launch_update_io<F32>(a, s);
}

}  // namespace ssm
