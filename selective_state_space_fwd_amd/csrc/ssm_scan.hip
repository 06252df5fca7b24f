// ssm_scan.hip -- selective-scan prefill kernels for gfx950.
//
// Sources (web pages on the Mamba selective scan):
//   ufo.work article "Mamba hardware-aware operator fusion and selective-scan
//     parallelisation" -- §1.1 recurrence and discretisation, §2.1 fusion of
//     every element-wise step into one kernel, §3.1 chunking with transfer
//     operators and a combine across chunks, §3.2 state-dimension groups,
//     §3.3 batch parallelism;
//   "From FlashAttention to Mamba" (kj168168) -- §三.2 prefix-scan form;
//   SSM engineering essay (discosf.com) -- §1.1 skip term D, §1.3 softplus
//     step size.
//
// Mapping on CDNA4.  One lane owns one channel (b, d) and one group of 16
// states, held in VGPRs; a wavefront covers 64 consecutive channels of one
// batch row.  Because A is diagonal, each lane runs the recurrence
// h = exp(dt A) h + dt B u serially over its tokens: no per-token scan work.
// Parallelism comes from channels, from state groups (a workgroup holds the
// G = ceil(N/16) groups of the same 64 channels, one wavefront each, and sums
// their partial C.h in LDS in a fixed order), and -- when channels are too
// few to fill 256 CUs -- from sequence chunks of K tokens:
//   pass 1 (chunk_kernel<AGG>)   every chunk but the last runs from a zero
//                                state; it publishes its transfer operator
//                                (sum of dt, h_end): A_chunk = exp(A sum dt),
//                                B_chunk = h_end;
//   pass 2 (carry_kernel)        an exclusive scan of the operators with the
//                                associative composition
//                                (a2,b2) o (a1,b1) = (a1 a2, a2 b1 + b2),
//                                lanes along chunks, wave64 DPP steps;
//   pass 3 (chunk_kernel<FULL>)  every chunk re-runs from its h_start and
//                                writes y (and the last chunk, last_state).
// B and C are shared by all channels of a batch row.  A pre-pass repacks them
// as fp32 rows [B_t(16) C_t(16)] per (b, t, group) so that a wavefront reads
// the 32 values of token t through scalar loads (one s_load_dwordx16 pair)
// and feeds them to the VALU as SGPR operands: no LDS traffic for B/C.
// u, delta and z (L-contiguous rows) are staged through LDS with coalesced
// loads and read back transposed, one row per lane.
#include "ssm_common.h"
#include "ssm_launch.h"

namespace ssm {

// ============================================================ B/C repack
// bc[((b*L + t)*G + g)*32 + k]: k < 16 -> B[b, 16g+k, t], else C[b, 16g+k-16, t];
// states n >= N are zero.  Grid ceil(L/64) * G * batch (1-D), 256 threads.
template <class IO>
__global__ __launch_bounds__(256) void bc_pack_kernel(const typename IO::T *__restrict__ Bm,
                                                      const typename IO::T *__restrict__ Cm,
                                                      float *__restrict__ bc, int64_t L, int N,
                                                      int G) {
    __shared__ float tile[32][65];
    const int64_t tiles = (L + 63) / 64;
    const int64_t blk = blockIdx.x;
    const int g = static_cast<int>((blk / tiles) % G);
    const int64_t b = blk / (tiles * G);
    const int64_t t0 = (blk % tiles) * 64;
    for (int idx = threadIdx.x; idx < 32 * 64; idx += 256) {
        const int k = idx >> 6, tt = idx & 63;
        const int n = g * kGroup + (k & 15);
        const int64_t t = t0 + tt;
        float v = 0.0f;
        if (n < N && t < L) {
            const size_t off = (static_cast<size_t>(b) * N + n) * L + t;
            v = k < 16 ? IO::load(Bm, off) : IO::load(Cm, off);
        }
        tile[k][tt] = v;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 32 * 64; idx += 256) {
        const int tt = idx >> 5, k = idx & 31;
        const int64_t t = t0 + tt;
        if (t < L) bc[((static_cast<size_t>(b) * L + t) * G + g) * 32 + k] = tile[k][tt];
    }
}

// ============================================================ chunk kernel
// Grid (n_cblk * batch, J); block 64*G threads (wavefront g = state group g).
// Tokens of chunk j: [j*K, min((j+1)*K, L)).
template <class IO, int G, int T, bool FULL>
__global__ __launch_bounds__(64 * G) void chunk_kernel(ScanArgs a) {
    using IT = typename IO::T;
    constexpr int NT = 64 * G;
    constexpr int TP = T + 1;                       // padded row: conflict-free column reads
    __shared__ float s_dt[kWave * TP];              // step size, then (G == 1) y
    __shared__ float s_w[kWave * TP];               // step size * u
    __shared__ float s_y[G > 1 ? G * kWave * TP : 1];

    const IT *__restrict__ u = static_cast<const IT *>(a.u);
    const IT *__restrict__ dl = static_cast<const IT *>(a.delta);
    const IT *__restrict__ z = static_cast<const IT *>(a.z);
    IT *__restrict__ y = static_cast<IT *>(a.y);
    cfloat *bc = as_constant(a.bc);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int g = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t b = blockIdx.x / a.n_cblk;
    const int64_t j = blockIdx.y;
    const int64_t d0 = static_cast<int64_t>(blockIdx.x % a.n_cblk) * kWave;
    const int64_t d = d0 + lane;
    const bool lane_ok = d < a.D;
    const int64_t L = a.L;
    const int64_t t_begin = j * a.K;
    const int64_t t_end = t_begin + a.K < L ? t_begin + a.K : L;
    const int Npad = G * kGroup;

    // Per-lane constants: A[d, n] * log2(e) (zero for padded states).
    float A2[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
        const int n = g * kGroup + i;
        A2[i] = (lane_ok && n < a.N) ? a.A[d * a.N + n] * kLog2e : 0.0f;
    }
    // Initial state of this chunk.
    float h[kGroup];
    const size_t cd = (static_cast<size_t>(b) * a.D + (lane_ok ? d : 0)) * a.J + j;
    if (FULL && a.J > 1) {
        const float *hs = a.hstart + cd * Npad + g * kGroup;
#pragma unroll
        for (int i = 0; i < kGroup; ++i) h[i] = lane_ok ? hs[i] : 0.0f;
    } else {
#pragma unroll
        for (int i = 0; i < kGroup; ++i) h[i] = 0.0f;
    }
    float dt_sum = 0.0f;

    for (int64_t t0 = t_begin; t0 < t_end; t0 += T) {
        // (a) coalesced load of the tile [64 channels x T tokens]: consecutive
        //     threads read consecutive tokens of a row.
        for (int idx = tid; idx < kWave * T; idx += NT) {
            const int r = idx / T, c = idx % T;
            const int64_t dd = d0 + r, t = t0 + c;
            float dt = 0.0f, w = 0.0f;
            if (dd < a.D && t < t_end) {
                const size_t off = (static_cast<size_t>(b) * a.D + dd) * L + t;
                const float uu = IO::load(u, off);
                float x = IO::load(dl, off);
                if (a.delta_bias) x += a.delta_bias[dd];
                dt = a.softplus ? softplus_f32(x) : x;
                w = dt * uu;
            }
            s_dt[r * TP + c] = dt;
            s_w[r * TP + c] = w;
        }
        __syncthreads();

        // (b) the recurrence, one lane per channel; B/C rows via scalar loads,
        //     fetched one token ahead.  Padded tokens have dt = 0 and w = 0:
        //     h is unchanged.
        const int tcount = static_cast<int>(t_end - t0 < T ? t_end - t0 : T);
        cfloat *p = bc + ((static_cast<size_t>(b) * L + t0) * G + g) * 32;
        float Bc[kGroup], Cc[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            Bc[i] = p[i];
            Cc[i] = FULL ? p[kGroup + i] : 0.0f;
        }
        float dtc = s_dt[lane * TP], wc = s_w[lane * TP];
#pragma unroll 2
        for (int c = 0; c < tcount; ++c) {
            const int cn = c + 1 < tcount ? c + 1 : c;
            cfloat *pn = p + (cn - c) * G * 32;
            float Bn[kGroup], Cn[kGroup];
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                Bn[i] = pn[i];
                Cn[i] = FULL ? pn[kGroup + i] : 0.0f;
            }
            const float dtn = s_dt[lane * TP + cn], wn = s_w[lane * TP + cn];
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                const float dA = exp2_hw(dtc * A2[i]);
                h[i] = __builtin_fmaf(dA, h[i], wc * Bc[i]);
                if (FULL) acc = __builtin_fmaf(Cc[i], h[i], acc);
            }
            if (FULL) {
                if (G == 1) s_dt[lane * TP + c] = acc;
                else s_y[(g * kWave + lane) * TP + c] = acc;
            } else {
                dt_sum += dtc;
            }
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                Bc[i] = Bn[i];
                Cc[i] = Cn[i];
            }
            dtc = dtn;
            wc = wn;
            p = pn;
        }

        // (c) finalize y for the tile: sum of group partials (fixed order),
        //     skip term, gate, coalesced store.
        if (FULL) {
            __syncthreads();
            for (int idx = tid; idx < kWave * T; idx += NT) {
                const int r = idx / T, c = idx % T;
                const int64_t dd = d0 + r, t = t0 + c;
                if (dd < a.D && t < t_end) {
                    float acc;
                    if (G == 1) {
                        acc = s_dt[r * TP + c];
                    } else {
                        acc = s_y[r * TP + c];
#pragma unroll
                        for (int gg = 1; gg < G; ++gg) acc += s_y[(gg * kWave + r) * TP + c];
                    }
                    const size_t off = (static_cast<size_t>(b) * a.D + dd) * L + t;
                    if (a.Dskip) acc = __builtin_fmaf(a.Dskip[dd], IO::load(u, off), acc);
                    if (a.z) acc *= silu_f32(IO::load(z, off));
                    IO::store(y, off, acc);
                }
            }
        }
        __syncthreads();
    }

    if (!lane_ok) return;
    if (FULL) {
        if (a.last_state && j == a.J - 1) {
            float *ls = a.last_state + (static_cast<size_t>(b) * a.D + d) * a.N;
#pragma unroll
            for (int i = 0; i < kGroup; ++i)
                if (g * kGroup + i < a.N) ls[g * kGroup + i] = h[i];
        }
    } else {
        float *he = a.hend + cd * Npad + g * kGroup;
#pragma unroll
        for (int i = 0; i < kGroup; ++i) he[i] = h[i];
        if (g == 0) a.dtsum[cd] = dt_sum;
    }
}

// ============================================================ carry kernel
// Exclusive scan of chunk transfer operators along the sequence, one
// wavefront per (b, d, state group), lanes along chunks (64 chunks per step).
// Lane j holds (a, b) = (exp(A sum_dt_j), h_end_j) for its 16 states.  The
// inclusive scan uses the DPP steps row_shr:1,2,4,8 (within rows of 16
// lanes), row_bcast:15 and row_bcast:31 (across rows); a lane whose source is
// out of range keeps the identity (1, 0).  wave_shr:1 makes it exclusive.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp(float old, float src) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src),
                                                      CTRL, ROWMASK, 0xF, false));
}

template <int CTRL, int ROWMASK>
__device__ __forceinline__ void scan_step(float &a, float &b) {
    // (a, b) := (a_prev, b_prev) then (a, b)
    const float ap = dpp<CTRL, ROWMASK>(1.0f, a);
    const float bp = dpp<CTRL, ROWMASK>(0.0f, b);
    b = __builtin_fmaf(a, bp, b);
    a = a * ap;
}

__global__ __launch_bounds__(256) void carry_kernel(ScanArgs a) {
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    const int G = a.G;
    const int64_t total = a.Bsz * a.D * G;
    if (wave >= total) return;                       // whole wavefront exits together
    const int g = static_cast<int>(wave % G);
    const int64_t bd = wave / G;                      // b * D + d
    const int64_t d = bd % a.D;
    const int Npad = G * kGroup;

    float A2[kGroup], hin[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
        const int n = g * kGroup + i;
        A2[i] = n < a.N ? a.A[d * a.N + n] * kLog2e : 0.0f;
        hin[i] = 0.0f;
    }
    for (int64_t j0 = 0; j0 < a.J; j0 += kWave) {
        const int64_t jj = j0 + lane;
        const bool ok = jj < a.J;                    // h_start is written for every chunk
        const bool has_op = jj < a.J - 1;            // the last chunk acts as identity
        const size_t cd = static_cast<size_t>(bd) * a.J + (ok ? jj : 0);
        const float sdt = has_op ? a.dtsum[cd] : 0.0f;
        const float *he = a.hend + cd * Npad + g * kGroup;
        float *hs = a.hstart + cd * Npad + g * kGroup;
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            float av = has_op ? exp2_hw(A2[i] * sdt) : 1.0f;
            float bv = has_op ? he[i] : 0.0f;
            scan_step<0x111, 0xF>(av, bv);   // row_shr:1
            scan_step<0x112, 0xF>(av, bv);   // row_shr:2
            scan_step<0x114, 0xF>(av, bv);   // row_shr:4
            scan_step<0x118, 0xF>(av, bv);   // row_shr:8
            scan_step<0x142, 0xA>(av, bv);   // row_bcast:15 -> rows 1, 3
            scan_step<0x143, 0xC>(av, bv);   // row_bcast:31 -> rows 2, 3
            // exclusive prefix: value of lane - 1, identity at lane 0
            const float ae = dpp<0x138, 0xF>(1.0f, av);   // wave_shr:1
            const float be = dpp<0x138, 0xF>(0.0f, bv);
            if (ok) hs[i] = __builtin_fmaf(ae, hin[i], be);
            // state after the last chunk of this step, for the next step
            const float a63 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(av), 63));
            const float b63 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 63));
            hin[i] = __builtin_fmaf(a63, hin[i], b63);
        }
    }
}

// ============================================================ zero fill
__global__ __launch_bounds__(256) void fill_zero_kernel(float *p, size_t n) {
    const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// ============================================================ launchers
template <class IO, int G>
static hipError_t launch_chunks(const ScanArgs &a, hipStream_t s) {
    constexpr int T = G == 1 ? 32 : 16;
    const dim3 grid(static_cast<unsigned>(a.n_cblk * a.Bsz), static_cast<unsigned>(a.J));
    if (a.J > 1) {
        // the last chunk's operator is never needed
        const dim3 agrid(static_cast<unsigned>(a.n_cblk * a.Bsz), static_cast<unsigned>(a.J - 1));
        hipLaunchKernelGGL((chunk_kernel<IO, G, T, false>), agrid, dim3(64 * G), 0, s, a);
        const int64_t waves = a.Bsz * a.D * a.G;
        const unsigned blocks = static_cast<unsigned>((waves + 3) / 4);
        hipLaunchKernelGGL(carry_kernel, dim3(blocks), dim3(256), 0, s, a);
    }
    if (a.ev_begin && a.ev_end) (void)hipEventRecord(a.ev_begin, s);
    hipLaunchKernelGGL((chunk_kernel<IO, G, T, true>), grid, dim3(64 * G), 0, s, a);
    if (a.ev_begin && a.ev_end) (void)hipEventRecord(a.ev_end, s);
    return hipGetLastError();
}

template <class IO>
static hipError_t launch_scan_io(const ScanArgs &a, hipStream_t s) {
    const dim3 pgrid(static_cast<unsigned>((a.L + 63) / 64 * a.G * a.Bsz));
    hipLaunchKernelGGL(bc_pack_kernel<IO>, pgrid, dim3(256), 0, s,
                       static_cast<const typename IO::T *>(a.B),
                       static_cast<const typename IO::T *>(a.C), a.bc, a.L, a.N, a.G);
    switch (a.G) {   // the plan pads G to a power of two
        case 1: return launch_chunks<IO, 1>(a, s);
        case 2: return launch_chunks<IO, 2>(a, s);
        case 4: return launch_chunks<IO, 4>(a, s);
        case 8: return launch_chunks<IO, 8>(a, s);
        case 16: return launch_chunks<IO, 16>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_scan(const ScanArgs &a, hipStream_t s) {
    return a.bf16 ? launch_scan_io<BF16>(a, s) : launch_scan_io<F32>(a, s);
}

hipError_t launch_fill_zero(float *p, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                       0, s, p, n);
    return hipGetLastError();
}

}  // namespace ssm
