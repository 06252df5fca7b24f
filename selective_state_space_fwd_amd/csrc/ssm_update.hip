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
// of P lanes (a fixed order).
#include "ssm_common.h"
#include "ssm_launch.h"

namespace ssm {

// 4 consecutive values of a row, one vector load (16 bytes fp32, 8 bf16).
template <class IO>
__device__ __forceinline__ void load4(const typename IO::T *p, float (&o)[4]);
template <>
__device__ __forceinline__ void load4<F32>(const float *p, float (&o)[4]) {
    const float4 v = *reinterpret_cast<const float4 *>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
template <>
__device__ __forceinline__ void load4<BF16>(const uint16_t *p, float (&o)[4]) {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
}

typedef float f4v __attribute__((ext_vector_type(4)));

// Coalesced path (N % 4 == 0, 16-byte aligned state and A): every thread
// serves ITER channels, 256 / P channels apart, and issues all their loads
// before any arithmetic, so ITER 16-byte state pieces per lane are in flight
// at once (the step is bound by bytes in flight over HBM latency).  The state
// is read and written with non-temporal accesses.
template <class IO, int ITER>
__global__ __launch_bounds__(256) void update_vec_kernel(UpdateArgs a, int P, int log2P) {
    using IT = typename IO::T;
    const IT *__restrict__ u = static_cast<const IT *>(a.u);
    const IT *__restrict__ dl = static_cast<const IT *>(a.delta);
    const IT *__restrict__ z = static_cast<const IT *>(a.z);
    const IT *__restrict__ Bm = static_cast<const IT *>(a.B);
    const IT *__restrict__ Cm = static_cast<const IT *>(a.C);
    IT *__restrict__ y = static_cast<IT *>(a.y);
    const int per_block = 256 >> log2P;              // channels per block and iteration
    const int l = threadIdx.x & (P - 1);
    const int n0 = 4 * l;
    const bool lane_on = n0 < a.N;                   // P * 4 may exceed N
    const int n0c = lane_on ? n0 : static_cast<int>(a.N) - 4;   // loads stay in the row
    const int64_t total = a.Bsz * a.D;
    const int64_t base = static_cast<int64_t>(blockIdx.x) * per_block * ITER + (threadIdx.x >> log2P);

    float4 sv[ITER], A4[ITER];
    float bv[ITER][4], cv[ITER][4], dt[ITER], uu[ITER], dk[ITER], zk[ITER];
#pragma unroll
    for (int k = 0; k < ITER; ++k) {
        const int64_t ch = base + static_cast<int64_t>(k) * per_block;
        const int64_t chs = ch < total ? ch : total - 1;   // clamped: loads stay in bounds
        const int64_t b = chs / a.D, d = chs % a.D;
        {
            // the state is touched once per step: stream it past the caches
            const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v *>(a.state + chs * a.N + n0c));
            sv[k] = make_float4(v.x, v.y, v.z, v.w);
        }
        A4[k] = *reinterpret_cast<const float4 *>(a.A + d * a.N + n0c);
        const size_t bo = static_cast<size_t>(b) * a.N + n0c;
        load4<IO>(Bm + bo, bv[k]);
        load4<IO>(Cm + bo, cv[k]);
        uu[k] = IO::load(u, chs);
        dt[k] = IO::load(dl, chs);
        // D and z too, with the rest: the output step then waits for no
        // second round trip to memory
        dk[k] = a.Dskip ? a.Dskip[d] : 0.0f;
        zk[k] = a.z ? IO::load(z, chs) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < ITER; ++k) {
        const int64_t ch = base + static_cast<int64_t>(k) * per_block;
        const bool ok = ch < total;                  // whole P-lane groups agree
        const int64_t chs = ok ? ch : total - 1;
        const float w = dt[k] * uu[k];
        float s4[4] = {sv[k].x, sv[k].y, sv[k].z, sv[k].w};
        const float av[4] = {A4[k].x, A4[k].y, A4[k].z, A4[k].w};
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float xa = dt[k] * (av[i] * kLog2e);
            const float dA = exp2_hw(xa);
            const float wi = a.zoh ? w * zoh_phi(xa * kLn2, dA) : w;
            s4[i] = __builtin_fmaf(dA, s4[i], wi * bv[k][i]);
            acc = __builtin_fmaf(cv[k][i], s4[i], acc);
        }
        if (ok && lane_on) {
            const f4v v = {s4[0], s4[1], s4[2], s4[3]};
            __builtin_nontemporal_store(v, reinterpret_cast<f4v *>(a.state + chs * a.N + n0));
        }
        if (!lane_on) acc = 0.0f;
        for (int off = P >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
        if (ok && l == 0) {
            if (a.Dskip) acc = __builtin_fmaf(dk[k], uu[k], acc);
            if (a.z) acc *= silu_f32(zk[k]);
            IO::store(y, chs, acc);
        }
    }
}

// General path: any N and alignment; one channel per P lanes.
template <class IO>
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
    // Sum over the P lanes of the channel (butterfly; fixed order per lane).
    for (int off = P >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (ok && l == 0) {
        if (a.Dskip) acc = __builtin_fmaf(a.Dskip[d], uu, acc);
        if (a.z) acc *= silu_f32(IO::load(z, chs));
        IO::store(y, chs, acc);
    }
}

// Channels per lane group of update_vec_kernel: two on large grids, where
// fewer, longer-lived wavefronts stream the state best; one on small grids,
// where twice the wavefronts shorten each lane's serial work.  Measured on
// MI355X (fp32, N = 16, gate): 256 x 5120 channels 32.9 us with two against
// 34.2 us with one; 16 x 5120: 4.52 against 4.29 us; 2 x 1536: 4.13 against
// 3.92 us.
constexpr int64_t kUpdateBigGrid = 2048;   // workgroups at two channels per lane group

template <class IO>
static hipError_t launch_update_io(const UpdateArgs &a, hipStream_t s) {
    const int groups = static_cast<int>((a.N + 3) / 4);
    int P = 1, log2P = 0;
    while (P < groups) { P <<= 1; ++log2P; }
    const int64_t channels = a.Bsz * a.D;
    auto al = [](const void *p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; };
    const uintptr_t bcal = a.bf16 ? 8 : 16;            // 4 elements of B and C
    const bool vec = (a.N % 4 == 0) && al(a.state, 16) && al(a.A, 16) && al(a.B, bcal) &&
                     al(a.C, bcal);
    if (vec) {
        const int64_t per_block2 = (256 >> log2P) * 2;
        const int64_t blocks2 = (channels + per_block2 - 1) / per_block2;
        if (blocks2 >= kUpdateBigGrid) {
            hipLaunchKernelGGL((update_vec_kernel<IO, 2>), dim3(static_cast<unsigned>(blocks2)),
                               dim3(256), 0, s, a, P, log2P);
        } else {
            const int64_t per_block = 256 >> log2P;
            const unsigned blocks = static_cast<unsigned>((channels + per_block - 1) / per_block);
            hipLaunchKernelGGL((update_vec_kernel<IO, 1>), dim3(blocks), dim3(256), 0, s, a, P,
                               log2P);
        }
    } else {
        const unsigned blocks = static_cast<unsigned>((channels * P + 255) / 256);
        hipLaunchKernelGGL((update_kernel<IO>), dim3(blocks), dim3(256), 0, s, a, P, log2P);
    }
    return hipGetLastError();
}

hipError_t launch_update(const UpdateArgs &a, hipStream_t s) {
    return a.bf16 ? launch_update_io<BF16>(a, s) : launch_update_io<F32>(a, s);
}

}  // namespace ssm
