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
// Mapping on CDNA4.  Because A is diagonal, every (channel, state) pair runs
// the recurrence h = exp(dt A) h + dt B u serially over its tokens, in a VGPR
// of one lane: no per-token scan work.  Two kernels share that core; both
// give a wavefront 16 channels in 4 lane-rows of 16 lanes:
//   quad_kernel   (d_state <= 16) 4 states per lane, one wavefront per block
//                 of 16 channels;
//   group_kernel  (16 < d_state <= 256) 8 states per lane, so 32 states per
//                 wavefront and G = ceil(N/32) wavefronts per workgroup, whose
//                 partial C.h are summed in LDS in a fixed order.
// The row-partials of C.h inside a wavefront are summed with cross-lane
// permutes.  B and C are shared by all channels of a batch row; they are read
// in place, as 16 (or 32 G) more rows of the tile, and kept state-major in
// LDS.  When channels are too few to fill 256 CUs, the sequence is also cut
// into chunks of K tokens:
//   pass 1 (<FULL = false>)      every chunk but the last runs from a zero
//                                state; it publishes its transfer operator
//                                (sum of dt, h_end): A_chunk = exp(A sum dt),
//                                B_chunk = h_end;
//   pass 2 (carry_kernel)        an exclusive scan of the operators with the
//                                associative composition
//                                (a2,b2) o (a1,b1) = (a1 a2, a2 b1 + b2),
//                                lanes along chunks, wave64 DPP steps -- or,
//                                when the chunks are few, each chunk of
//                                pass 3 folds its predecessors itself;
//   pass 3 (<FULL = true>)       every chunk re-runs from its h_start and
//                                writes y (and the last chunk, last_state).
#include <type_traits>

#include <hip/hip_ext.h>

#include "ssm_common.h"
#include "ssm_launch.h"
#include "ssm_seq.h"

namespace ssm {

// Lane n of each 16-lane row, broadcast to the whole row (gfx90a+ DPP).
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + N, 0xF, 0xF, true));
}

template <class IO>
struct Piece4;   // 4 consecutive tokens of a row: 16 bytes (fp32) or 8 bytes (bf16)

template <>
struct Piece4<F32> {
    using V = float4;
    static __device__ __forceinline__ void unpack(const V &v, float (&o)[4]) {
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
    static __device__ __forceinline__ V pack(const float (&o)[4]) {
        return make_float4(o[0], o[1], o[2], o[3]);
    }
};

template <>
struct Piece4<BF16> {
    using V = uint2;
    static __device__ __forceinline__ void unpack(const V &v, float (&o)[4]) {
        o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
        o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
    }
    static __device__ __forceinline__ V pack(const float (&o)[4]) {
        // only ever packs values that were read from bf16 storage: exact
        return make_uint2((__float_as_uint(o[0]) >> 16) | (__float_as_uint(o[1]) & 0xffff0000u),
                          (__float_as_uint(o[2]) >> 16) | (__float_as_uint(o[3]) & 0xffff0000u));
    }
};


// The transfer operator's decay for chunk i of batch row b: exp(A sum dt),
// or 0 when a sequence starts inside the chunk.
__device__ __forceinline__ float chunk_decay(const ScanArgs &a, int64_t b, int64_t i, float A2,
                                             float sdt) {
    return a.keep[b * a.J + i] != 0.0f ? exp2_hw(A2 * sdt) : 0.0f;
}

// Final state of sequence s: states n0 .. n0 + S - 1 of channel d.
template <int S>
__device__ __forceinline__ void store_final_state(const ScanArgs &a, int64_t s, int64_t d,
                                                  bool lane_ok, int n0, const float (&h)[S]) {
    if (!a.last_state || !lane_ok) return;
    float *ls = a.last_state + (s * a.D + d) * a.N;
#pragma unroll
    for (int k = 0; k < S; ++k)
        if (n0 + k < a.N) ls[n0 + k] = h[k];
}

// ============================================================ causal convolution
// The short depthwise convolution ahead of the scan ("From FlashAttention to
// Mamba", §三.3), for NT consecutive tokens t .. t + NT - 1 of one channel
// row.  The raw inputs are in LDS at xs[-3 .. NT) (xs[i] = x_{t+i}); cw holds
// the weights of x_{t-3} .. x_t (zero for taps beyond the width).  Inputs
// before the sequence start of a token come from conv_state, or are zero.
template <int NT, bool EXT>
__device__ __forceinline__ void conv_run(const ScanArgs &a, const float *xs, int64_t t,
                                         const SeqPos &sp, int64_t st_cur, int64_t drc,
                                         float4 cw, float cb, float (&u)[NT]) {
    float xv[NT + 3];
#pragma unroll
    for (int m = 0; m < NT + 3; ++m) xv[m] = xs[m - 3];
    const int W = a.conv_w;
    const float wk[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int64_t tt = t + i;
        int64_t s = sp.s, st = st_cur;
        // a later packed sequence (padding tokens past L belong to the last
        // one); without packed sequences every token shares the row's start
        if (EXT && a.cu && tt >= sp.end) {
            s = seq_of(a, tt);
            st = cu_at(a, s);
        }
        float acc = cb;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t src = tt - 3 + k;
            float v = xv[i + k];
            if (k < 4 - W) {
                v = 0.0f;
            } else if (src < st) {
                v = a.conv_state
                        ? a.conv_state[(s * a.D + drc) * (W - 1) + (W - 1) - (st - src)]
                        : 0.0f;
            }
            acc = __builtin_fmaf(wk[k], v, acc);
        }
        u[i] = a.conv_silu ? silu_f32(acc) : acc;
    }
}

// Weights of one channel as the 4 taps on x_{t-3} .. x_t.
__device__ __forceinline__ float4 conv_taps(const ScanArgs &a, int64_t drc) {
    const int W = a.conv_w;
    float w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int kk = k - (4 - W);
        w[k] = kk >= 0 ? a.conv_weight[drc * W + (kk >= 0 ? kk : 0)] : 0.0f;
    }
    return make_float4(w[0], w[1], w[2], w[3]);
}

// One token of the recurrence for one state: h = exp(dt A) h + c B u, with
// w_b = dt u B and c the Euler factor 1 or, under zero-order hold, phi(dt A).
// A2 = A log2(e), so dt A2 feeds the base-2 exponential directly.
template <bool ZOH>
__device__ __forceinline__ float state_step(float dt, float A2, float h, float w_b) {
    const float xa = dt * A2;
    const float e = exp2_hw(xa);
    return __builtin_fmaf(e, h, ZOH ? w_b * zoh_phi(xa * kLn2, e) : w_b);
}

// ============================================================ quad-row kernel (N <= 16)
// The path for d_state <= 16.  A wavefront covers 16 channels in 4 lane-rows:
// lane l serves channel c = l % 16 and the 4 states 4q..4q+3, q = l / 16.
// Compared with one lane per channel this streams 16 rows per wavefront
// instead of 64 (the partially consumed cache lines of all wavefronts in
// flight then fit in the L2 of their XCD, so each line is fetched once), and
// it gives 4x as many wavefronts, so fewer sequence chunks are needed to fill
// the chip.  Per 4 tokens the 4 row-partials of C.h are summed with a
// transposing butterfly of v_permlane16_swap / v_permlane32_swap (3 swaps and
// 3 adds): afterwards row q holds the full sum for token q of the group.
//
// Tile: 16 channels x T tokens, T = 64 bytes / element size.  B and C keep
// their (batch, N, L) layout, so the tile's B rows (and C rows) are 16 more
// rows of the same shape as the channel rows: every lane loads exactly one
// 16-byte piece of each of u, delta, z, B and C per tile, one tile ahead.
// Per tile:
//  (a) convert the lane's pieces (dt = softplus(delta + bias), w = dt u,
//      du = D u; B and C widened to fp32, states n >= N zeroed) into LDS
//      rows padded to T + 4 floats; g = silu(z) stays in the lane's VGPRs;
//  (b) walk the tile 4 tokens at a time.  ds_read_b128 gives 4 tokens of
//      dt, of w and of B[4q + (lane % 4)]; B_t[4q + k] enters w B through
//      the DPP operand row_newbcast:k (lane 16q + k holds state 4q + k), and
//      C[4q + k] for 4 tokens is one more ds_read_b128 per state;
//  (c) y = (C h + D u) g from the LDS row and the lane's g, coalesced
//      16-byte stores.
// A FULL pass that starts inside the sequence takes its start state either
// from the carry kernel (h_start) or, when the chunks before it are few, by
// folding their transfer operators itself: h = exp(A sum dt) h + h_end, in
// chunk order.
// EXT: the instance that also handles packed sequences and the fused
// convolution; calls with neither use the lean instance.  ZOH (EXT only):
// zero-order-hold input term.
//
// quad_pass runs one chunk j of one 16-channel block; the kernels below
// call it.  FULL = false: the chunk-aggregate pass, which leaves the chunk's
// end state (from zero, or from the start state of a sequence that begins
// in it) in h, its sum of dt in dt_sum and its keep flag in keep.  FULL =
// true: the pass that writes y and final states; with GIVEN it starts from
// the state the caller leaves in h (unless a sequence starts at its first
// token), else from h_start or the fold of the workspace operators.
// The LDS tiles are the caller's, as distinct restrict-qualified arrays, so
// that the compiler sees that the y written by one token group (into s_du,
// in place) never aliases the dt, w, B and C read by the next group, and
// can issue those reads early.
template <class IO, bool FULL>
struct QuadTile {
    static constexpr int VW = Seg<IO>::VW;
    static constexpr int T = 4 * VW;                // 64 bytes of a row per tile
    static constexpr int TP = T + 4;
    static constexpr int QC = 16;                   // channels per wavefront
    static constexpr int n_dt = QC * TP;
    // s_w rows start 4 floats in: the 4 floats before a row's tokens (the
    // previous row's padding) keep the inputs of the 4 tokens before the
    // tile when the scan input is computed by the causal convolution
    static constexpr int n_w = QC * TP + 4;
    static constexpr int n_du = FULL ? QC * TP : 4;   // D u, then y
    static constexpr int n_B = 16 * TP;               // state-major
    static constexpr int n_C = FULL ? 16 * TP : 4;
};

// Token range of chunk j on the uniform chunking: j K .. min(j K + K, L).
__device__ __forceinline__ int64_t chunk_end(const ScanArgs &a, int64_t j) {
    return j * a.K + a.K < a.L ? j * a.K + a.K : a.L;
}

// FAIR: fair_prio on every tile (the two-pass kernels; the one-launch
// kernel sets its own priorities).
// blk: the 16-channel block (batch row blk / n_cblk); chunk j covers tokens
// t_begin .. t_end - 1 (j K .. min(j K + K, L) on the uniform chunking).
template <class IO, bool FULL, bool VEC, bool EXT, bool ZOH, bool GIVEN, bool FAIR = false>
__device__ __forceinline__ void quad_pass(const ScanArgs &a, int64_t blk, int64_t j,
                                          int64_t t_begin, int64_t t_end, float (&h)[4],
                                          float &dt_sum_out, float &keep_out,
                                          float *__restrict__ s_dt, float *__restrict__ s_w,
                                          float *__restrict__ s_du,
                                          float *__restrict__ s_B, float *__restrict__ s_C) {
    using IT = typename IO::T;
    using S = Seg<IO>;
    using V = typename S::V;
    constexpr int VW = S::VW;
    constexpr int T = 4 * VW;                       // 64 bytes of a row per tile
    constexpr int TP = T + 4;
    constexpr int QC = 16;                          // channels per wavefront

    const IT *__restrict__ u = static_cast<const IT *>(a.u);
    const IT *__restrict__ dl = static_cast<const IT *>(a.delta);
    const IT *__restrict__ z = static_cast<const IT *>(a.z);
    const IT *__restrict__ Bm = static_cast<const IT *>(a.B);
    const IT *__restrict__ Cm = static_cast<const IT *>(a.C);
    IT *__restrict__ y = static_cast<IT *>(a.y);

    const int lane = threadIdx.x;
    const int c = lane & 15;                        // channel within the block
    const int q = lane >> 4;                        // lane-row: states 4q .. 4q+3
    const int64_t b = blk / a.n_cblk;
    const int64_t d0 = static_cast<int64_t>(blk % a.n_cblk) * QC;
    const int64_t d = d0 + c;
    const bool lane_ok = d < a.D;
    const int64_t L = a.L;
    const bool gate = a.z != nullptr;

    // ---- this lane's tile pieces: row r (channel d0 + r, and state r of B
    // and C), tokens [sc, sc + VW) of the tile
    const int r = lane >> 2;
    const int sc = (lane & 3) * VW;
    const int64_t dr = d0 + r;
    const bool row_ok = dr < a.D;
    const bool rows_full = d0 + QC <= a.D;          // wave-uniform
    const int64_t drc = row_ok ? dr : a.D - 1;
    const size_t rbase = (static_cast<size_t>(b) * a.D + drc) * L;
    const float rbias = (row_ok && a.delta_bias) ? a.delta_bias[drc] : 0.0f;
    const float rD = (row_ok && a.Dskip) ? a.Dskip[drc] : 0.0f;
    const bool st_ok = r < a.N;
    const size_t sbase = (static_cast<size_t>(b) * a.N + (st_ok ? r : a.N - 1)) * L;
    const bool conv = EXT && a.conv_w > 0;                 // u holds the convolution's input
    const float4 cw = conv ? conv_taps(a, drc) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float cbias = (conv && a.conv_bias) ? a.conv_bias[drc] : 0.0f;

    // Prefetched tile registers: named vectors only (no arrays or aggregates
    // carried around the loop), so that they stay in VGPRs.
    V vu{}, vd{}, vz{}, vb{}, vc{};
    // element path: VW scalar loads per tensor, packed into the same vector
    // registers as the 16-byte path; tokens past the chunk are clamped to its
    // last token (their values are never used)
    auto load_elems = [&](const IT *p, size_t base, int64_t t) {
        float e[VW];
#pragma unroll
        for (int i = 0; i < VW; ++i) {
            const int64_t tc = t + i < t_end ? t + i : t_end - 1;
            e[i] = IO::load(p, base + tc);
        }
        return S::pack(e);
    };
    // VIEWS: the tile loads and the y and checkpoint stores go through
    // wave-uniform buffer views: the block's rows of u, delta, z and y (up to
    // 16 channels of L elements), the batch row's N rows of B and C (rows
    // r >= N read as zeros) and the block's checkpoint rows.  A lane's piece
    // of row r lies at r L elements plus its token.  Loads past a chunk's end
    // read the next tokens (masked in the walk), past the view zeros; a store
    // that must not happen aims past its view (kDrop) and is dropped, so the
    // stores are the same instructions on every path and the compiler's
    // count of memory operations in flight stays exact (a store under a
    // branch makes the wait for the next tile's loads wait for it too).
    // The packed-sequence / convolution instance (EXT without ZOH) keeps
    // plain pointers: there the views' scalar registers spilled (25 -> 59
    // SGPRs) and it ran slower (Mamba-2.8B-shaped layer packed as 5
    // sequences 698 -> 736 us, with the fused convolution 498 -> 509 us;
    // with zero-order hold 865 -> 800 us, which keeps them).
    constexpr bool VIEWS = VEC && (!EXT || ZOH);
    constexpr uint32_t ESZ = sizeof(IT);
    const int64_t d0v = d0 < a.D ? d0 : a.D - 1;
    const int64_t nrows = a.D - d0v < QC ? a.D - d0v : QC;
    const size_t blk0 = (static_cast<size_t>(b) * a.D + d0v) * L;
    const uint64_t blk_bytes = VIEWS ? static_cast<uint64_t>(nrows) * L * ESZ : 0;
    const Rsrc v_u = view(u + blk0, blk_bytes), v_d = view(dl + blk0, blk_bytes);
    const Rsrc v_z = view((gate ? z : u) + blk0, blk_bytes);
    const Rsrc v_y = view(y ? y + blk0 : u + blk0, FULL && y ? blk_bytes : 0);
    const uint64_t bc_bytes = VIEWS ? static_cast<uint64_t>(a.N) * L * ESZ : 0;
    const Rsrc v_b = view(Bm + static_cast<size_t>(b) * a.N * L, bc_bytes);
    const Rsrc v_c = view(Cm + static_cast<size_t>(b) * a.N * L, bc_bytes);
    const uint32_t o_row = static_cast<uint32_t>(r) * static_cast<uint32_t>(L) * ESZ;
    auto load_view = [&](Rsrc v, uint32_t off) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(v, off, 0, 0);
        V o;
        if constexpr (std::is_same<IO, F32>::value) {
            o = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]),
                            __uint_as_float(x[3]));
        } else {
            o = make_uint4(x[0], x[1], x[2], x[3]);
        }
        return o;
    };
    auto load_tile = [&](int64_t t0) {
        const int64_t t = t0 + sc;
        if constexpr (VIEWS) {
            const uint32_t off = o_row + static_cast<uint32_t>(t) * ESZ;
            vu = load_view(v_u, off);
            vd = load_view(v_d, off);
            if (FULL && gate) vz = load_view(v_z, off);
            vb = load_view(v_b, off);
            if (FULL) vc = load_view(v_c, off);
        } else if constexpr (VEC) {
            const int64_t tc = t < t_end ? t : t_end - VW;   // t_end >= VW here
            vu = *reinterpret_cast<const V *>(u + rbase + tc);
            vd = *reinterpret_cast<const V *>(dl + rbase + tc);
            if (FULL && gate) vz = *reinterpret_cast<const V *>(z + rbase + tc);
            vb = *reinterpret_cast<const V *>(Bm + sbase + tc);
            if (FULL) vc = *reinterpret_cast<const V *>(Cm + sbase + tc);
        } else {
            vu = load_elems(u, rbase, t);
            vd = load_elems(dl, rbase, t);
            if (FULL && gate) vz = load_elems(z, rbase, t);
            vb = load_elems(Bm, sbase, t);
            if (FULL) vc = load_elems(Cm, sbase, t);
        }
    };

    // ---- per-lane constants and initial state
    const int64_t dcl = lane_ok ? d : a.D - 1;
    float A2[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int n = 4 * q + k;
        const float v = a.A[dcl * a.N + (n < a.N ? n : a.N - 1)];
        A2[k] = (lane_ok && n < a.N) ? v * kLog2e : 0.0f;
    }
    const size_t cd0 = (static_cast<size_t>(b) * a.D + dcl) * a.J;   // chunk 0 of this channel
    const size_t cd = cd0 + j;
    SeqPos sp = seq_pos<EXT>(a, b, t_begin);
    // the chunk's operator ignores its incoming state if a sequence starts in it
    keep_out = (!sp.reset && sp.end >= t_end) ? 1.0f : 0.0f;
    load_tile(t_begin);
    if (sp.reset) {
        load_start_state<4>(a, sp.s, dcl, lane_ok, 4 * q, h);
    } else if (!FULL) {
        h[0] = h[1] = h[2] = h[3] = 0.0f;
    } else if (GIVEN) {
        if (!lane_ok) h[0] = h[1] = h[2] = h[3] = 0.0f;
    } else {
        h[0] = h[1] = h[2] = h[3] = 0.0f;
        // a chunk after the first of its sequence: start from h_start
        if (a.hstart) {
            const float4 v = *reinterpret_cast<const float4 *>(a.hstart + cd * 16 + 4 * q);
            h[0] = v.x; h[1] = v.y; h[2] = v.z; h[3] = v.w;
        } else {
            // fold the transfer operators of chunks 0 .. j-1 in order
            for (int64_t i = 0; i < j; ++i) {
                const float sdt = a.dtsum[cd0 + i];
                const float4 v = *reinterpret_cast<const float4 *>(a.hend + (cd0 + i) * 16 + 4 * q);
                h[0] = __builtin_fmaf(chunk_decay(a, b, i, A2[0], sdt), h[0], v.x);
                h[1] = __builtin_fmaf(chunk_decay(a, b, i, A2[1], sdt), h[1], v.y);
                h[2] = __builtin_fmaf(chunk_decay(a, b, i, A2[2], sdt), h[2], v.z);
                h[3] = __builtin_fmaf(chunk_decay(a, b, i, A2[3], sdt), h[3], v.w);
            }
        }
        // padded channels carry no state (their A is zeroed, B is not)
        if (!lane_ok) h[0] = h[1] = h[2] = h[3] = 0.0f;
    }
    float dt_sum = 0.0f;
    if (conv && (lane & 3) == 0) {
        // convolution inputs of the 4 tokens before the chunk
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t tt = t_begin - 4 + k;
            s_w[r * TP + k] = tt >= 0 ? IO::load(u, rbase + tt) : 0.0f;
        }
    }
    // checkpoints for the backward pass: the state entering every
    // kBwdTile-token tile of the row (chunks start on such tiles)
    float *ckp = (FULL && a.ckpt && lane_ok)
                     ? a.ckpt + (static_cast<size_t>(b) * a.D + d) * a.n_ck * 16 + 4 * q
                     : nullptr;
    // VIEWS: the block's checkpoint rows as a view (empty without
    // checkpoints, so that every store is dropped); lane (channel c, row q)
    // writes floats 4q .. 4q+3 of entry c n_ck + t / kBwdTile (16 floats each)
    const Rsrc v_ck = view(a.ckpt ? a.ckpt + (static_cast<size_t>(b) * a.D + d0v) * a.n_ck * 16 : a.A,
                           (VIEWS && FULL && a.ckpt) ? static_cast<uint64_t>(nrows) * a.n_ck * 64 : 0);
    const uint32_t o_ck = (static_cast<uint32_t>(lane & 15) * static_cast<uint32_t>(a.n_ck) * 16 +
                           4 * q) * 4;
    // h is the state entering token t; `when` (uniform): the store happens
    auto ckpt_at = [&](int64_t t, bool when) {
        if constexpr (VIEWS) {
            using V4 = __attribute__((ext_vector_type(4))) unsigned int;
            const uint32_t off = when ? o_ck + static_cast<uint32_t>(t / kBwdTile) * 64 : kDrop;
            __builtin_amdgcn_raw_buffer_store_b128(
                V4{__float_as_uint(h[0]), __float_as_uint(h[1]), __float_as_uint(h[2]),
                   __float_as_uint(h[3])}, v_ck, off, 0, 0);
        } else {
            if (ckp && when)
                *reinterpret_cast<float4 *>(ckp + (t / kBwdTile) * 16) = make_float4(h[0], h[1], h[2], h[3]);
        }
    };
    if (FULL) ckpt_at(t_begin, true);

    // silu(z) (1 without a gate) of this lane's piece of the tile: the lane
    // that converts a piece is the one that stores its y, so the gate stays
    // in registers from (a) to (c)
    float gk[VW];
    const int64_t n_tiles = (t_end - t_begin + T - 1) / T;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += T) {
        if (FAIR) fair_prio((t0 - t_begin) / T, n_tiles);
        if (conv) {
            // (a0) the scan input u = act(conv(x)) of this lane's piece: stage
            // the raw inputs, convolve, keep the tile's last 4 inputs for the
            // next tile, and leave u in s_dt for the conversion below
            float xr[VW], uc[VW];
            S::unpack(vu, xr);
            const int o = r * TP + sc;
#pragma unroll
            for (int i = 0; i < VW; i += 4)
                *reinterpret_cast<float4 *>(&s_w[4 + o + i]) = make_float4(xr[i], xr[i + 1], xr[i + 2], xr[i + 3]);
            __syncthreads();
            const int64_t st_cur = (EXT && a.cu) ? cu_at(a, sp.s) : 0;
            conv_run<VW, EXT>(a, &s_w[4 + o], t0 + sc, sp, st_cur, drc, cw, cbias, uc);
            __syncthreads();
            if (sc == T - VW) {
#pragma unroll
                for (int k = 0; k < 4; ++k) s_w[r * TP + k] = xr[VW - 4 + k];
            }
#pragma unroll
            for (int i = 0; i < VW; i += 4)
                *reinterpret_cast<float4 *>(&s_dt[o + i]) = make_float4(uc[i], uc[i + 1], uc[i + 2], uc[i + 3]);
            if (FULL && a.u_out) {
                IT *uo = static_cast<IT *>(a.u_out);
                const int64_t t = t0 + sc;
                if (VEC) {
                    if (row_ok && t < t_end) *reinterpret_cast<V *>(uo + rbase + t) = S::pack(uc);
                } else {
#pragma unroll
                    for (int i = 0; i < VW; ++i)
                        if (row_ok && t + i < t_end) IO::store(uo, rbase + t + i, uc[i]);
                }
            }
        }
        // (a) convert this lane's pieces and write them to LDS
        auto convert = [&](auto sp_tag, auto gate_tag, auto mask_tag) {
            constexpr bool SP = decltype(sp_tag)::value;
            constexpr bool GT = decltype(gate_tag)::value;
            constexpr bool MASK = decltype(mask_tag)::value;
            float xu[VW], xd[VW], xz[VW];
            if (conv) {
                // the convolution left u in this lane's own s_dt slots
#pragma unroll
                for (int i = 0; i < VW; ++i) xu[i] = s_dt[r * TP + sc + i];
            } else {
                S::unpack(vu, xu);
            }
            S::unpack(vd, xd);
            if (FULL && GT) S::unpack(vz, xz);
            float xdt[VW], xw[VW], xdu[VW], xg[VW];
#pragma unroll
            for (int i = 0; i < VW; ++i) {
                // branch-free: evaluate for every lane, zero by a 0/1 factor
                // (only the last tile of a chunk or block needs the mask)
                const float m = !MASK || (row_ok && t0 + sc + i < t_end) ? 1.0f : 0.0f;
                const bool ok = !MASK || m != 0.0f;
                const float x = xd[i] + rbias;
                const float dt = MASK ? (SP ? softplus_f32(x) : x) * m : (SP ? softplus_f32(x) : x);
                const float uu = ok ? xu[i] : 0.0f;
                xdt[i] = dt;
                xw[i] = dt * uu;
                if (FULL) {
                    xdu[i] = rD * uu;
                    xg[i] = GT ? silu_f32(ok ? xz[i] : 0.0f) : 1.0f;
                }
            }
            const int o = r * TP + sc;
#pragma unroll
            for (int i = 0; i < VW; i += 4) {
                *reinterpret_cast<float4 *>(&s_dt[o + i]) = make_float4(xdt[i], xdt[i + 1], xdt[i + 2], xdt[i + 3]);
                *reinterpret_cast<float4 *>(&s_w[4 + o + i]) = make_float4(xw[i], xw[i + 1], xw[i + 2], xw[i + 3]);
                if (FULL) {
                    *reinterpret_cast<float4 *>(&s_du[o + i]) = make_float4(xdu[i], xdu[i + 1], xdu[i + 2], xdu[i + 3]);
                }
            }
            if (FULL) {
#pragma unroll
                for (int i = 0; i < VW; ++i) gk[i] = xg[i];
            }
        };
        using T_ = std::true_type;
        using F_ = std::false_type;
        if (rows_full && t0 + T <= t_end) {
            if (a.softplus) {
                if (FULL && gate) convert(T_{}, T_{}, F_{}); else convert(T_{}, F_{}, F_{});
            } else {
                if (FULL && gate) convert(F_{}, T_{}, F_{}); else convert(F_{}, F_{}, F_{});
            }
        } else {
            if (a.softplus) {
                if (FULL && gate) convert(T_{}, T_{}, T_{}); else convert(T_{}, F_{}, T_{});
            } else {
                if (FULL && gate) convert(F_{}, T_{}, T_{}); else convert(F_{}, F_{}, T_{});
            }
        }
        {
            // B and C rows: state r; states n >= N are zero
            float xb[VW], xc[VW];
            S::unpack(vb, xb);
            if (FULL) S::unpack(vc, xc);
            const int o = r * TP + sc;
#pragma unroll
            for (int i = 0; i < VW; i += 4) {
                // (VIEWS: rows past N read as zeros)
                const bool keep_bc = VIEWS || st_ok;
                *reinterpret_cast<float4 *>(&s_B[o + i]) =
                    keep_bc ? make_float4(xb[i], xb[i + 1], xb[i + 2], xb[i + 3])
                            : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                if (FULL)
                    *reinterpret_cast<float4 *>(&s_C[o + i]) =
                        keep_bc ? make_float4(xc[i], xc[i + 1], xc[i + 2], xc[i + 3])
                                : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        }
        // Unconditional prefetch (addresses are clamped into range): the same
        // number of loads on every path keeps the wait counts exact.
        load_tile(t0 + T);
        __syncthreads();

        // (b) the recurrence, 4 tokens per group.  The whole tile is one
        // straight-line block (tokens past the chunk end are no-ops: dt = 0,
        // w = 0), so the LDS reads of a group can be issued under the
        // previous group's math.
        const int rowc = c * TP;
        const int brow = (4 * q + (lane & 3)) * TP;   // B row-replication source
        const int crow = 4 * q * TP;
        if (EXT && sp.end < t0 + T && sp.end < t_end) {
            // a sequence boundary inside the tile: token by token
            for (int k = 0; k < T; ++k) {
                const int64_t t = t0 + k;
                if (t == sp.end && t < t_end) {
                    if (FULL) store_final_state<4>(a, sp.s, d, lane_ok, 4 * q, h);
                    sp = seq_pos<EXT>(a, b, t);
                    load_start_state<4>(a, sp.s, dcl, lane_ok, 4 * q, h);
                }
                const float dt = s_dt[rowc + k], w = s_w[4 + rowc + k], Bk = s_B[brow + k];
                h[0] = state_step<ZOH>(dt, A2[0], h[0], row_bcast<0>(Bk) * w);
                h[1] = state_step<ZOH>(dt, A2[1], h[1], row_bcast<1>(Bk) * w);
                h[2] = state_step<ZOH>(dt, A2[2], h[2], row_bcast<2>(Bk) * w);
                h[3] = state_step<ZOH>(dt, A2[3], h[3], row_bcast<3>(Bk) * w);
                if (FULL) {
                    float acc = s_C[crow + k] * h[0];
                    acc = __builtin_fmaf(s_C[crow + TP + k], h[1], acc);
                    acc = __builtin_fmaf(s_C[crow + 2 * TP + k], h[2], acc);
                    acc = __builtin_fmaf(s_C[crow + 3 * TP + k], h[3], acc);
                    acc += __shfl_xor(acc, 16);
                    acc += __shfl_xor(acc, 32);
                    if (q == 0) s_du[rowc + k] = acc + s_du[rowc + k];
                } else {
                    dt_sum += dt;
                }
                if (FULL && (t + 1) % kBwdTile == 0 && t + 1 < t_end) ckpt_at(t + 1, true);
            }
        } else {
#pragma unroll
        for (int c4 = 0; c4 < T; c4 += 4) {
            const float4 dt4 = *reinterpret_cast<const float4 *>(&s_dt[rowc + c4]);
            const float4 w4 = *reinterpret_cast<const float4 *>(&s_w[4 + rowc + c4]);
            const float4 B4 = *reinterpret_cast<const float4 *>(&s_B[brow + c4]);
            float4 C0{}, C1{}, C2{}, C3{};
            if (FULL) {
                C0 = *reinterpret_cast<const float4 *>(&s_C[crow + c4]);
                C1 = *reinterpret_cast<const float4 *>(&s_C[crow + TP + c4]);
                C2 = *reinterpret_cast<const float4 *>(&s_C[crow + 2 * TP + c4]);
                C3 = *reinterpret_cast<const float4 *>(&s_C[crow + 3 * TP + c4]);
            }
            const float dtv[4] = {dt4.x, dt4.y, dt4.z, dt4.w};
            const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
            const float bv[4] = {B4.x, B4.y, B4.z, B4.w};
            const float c0[4] = {C0.x, C0.y, C0.z, C0.w};
            const float c1[4] = {C1.x, C1.y, C1.z, C1.w};
            const float c2[4] = {C2.x, C2.y, C2.z, C2.w};
            const float c3[4] = {C3.x, C3.y, C3.z, C3.w};
            float accv[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float dt = dtv[k], w = wv[k], Bk = bv[k];
                h[0] = state_step<ZOH>(dt, A2[0], h[0], row_bcast<0>(Bk) * w);
                h[1] = state_step<ZOH>(dt, A2[1], h[1], row_bcast<1>(Bk) * w);
                h[2] = state_step<ZOH>(dt, A2[2], h[2], row_bcast<2>(Bk) * w);
                h[3] = state_step<ZOH>(dt, A2[3], h[3], row_bcast<3>(Bk) * w);
                if (FULL)
                    accv[k] = __builtin_fmaf(c0[k], h[0], __builtin_fmaf(c1[k], h[1],
                              __builtin_fmaf(c2[k], h[2], c3[k] * h[3])));
                else
                    dt_sum += dt;
            }
            if (FULL) {
                // rows (0,1) and (2,3): even rows sum token 0/2, odd rows 1/3
                const auto s01 = __builtin_amdgcn_permlane16_swap(
                    __float_as_uint(accv[0]), __float_as_uint(accv[1]), false, false);
                const auto s23 = __builtin_amdgcn_permlane16_swap(
                    __float_as_uint(accv[2]), __float_as_uint(accv[3]), false, false);
                const float p01 = __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
                const float p23 = __uint_as_float(s23[0]) + __uint_as_float(s23[1]);
                // halves: rows 0,1 keep tokens 0,1; rows 2,3 keep tokens 2,3
                const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(p01),
                                                                __float_as_uint(p23), false, false);
                const float ysum = __uint_as_float(s[0]) + __uint_as_float(s[1]);   // token c4 + q
                const int o = rowc + c4 + q;
                s_du[o] = ysum + s_du[o];
                if ((c4 + 4) % kBwdTile == 0) ckpt_at(t0 + c4 + 4, t0 + c4 + 4 < t_end);
            }
        }
        }

        // (c) coalesced store of y
        if (FULL) {
            __syncthreads();
            const int64_t t = t0 + sc;
            const int o = r * TP + sc;
            float yo[VW];
#pragma unroll
            for (int i = 0; i < VW; i += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(&s_du[o + i]);
                yo[i] = v.x * gk[i];
                yo[i + 1] = v.y * gk[i + 1];
                yo[i + 2] = v.z * gk[i + 2];
                yo[i + 3] = v.w * gk[i + 3];
            }
            if constexpr (VIEWS) {
                const typename S::V pv = S::pack(yo);
                using V4 = __attribute__((ext_vector_type(4))) unsigned int;
                V4 w;
                if constexpr (std::is_same<IO, F32>::value) {
                    w = V4{__float_as_uint(pv.x), __float_as_uint(pv.y), __float_as_uint(pv.z),
                           __float_as_uint(pv.w)};
                } else {
                    w = V4{pv.x, pv.y, pv.z, pv.w};
                }
                const uint32_t off = (row_ok && t < t_end) ? o_row + static_cast<uint32_t>(t) * ESZ : kDrop;
                __builtin_amdgcn_raw_buffer_store_b128(w, v_y, off, 0, 0);
            } else if constexpr (VEC) {
                if (row_ok && t < t_end)
                    *reinterpret_cast<typename S::V *>(y + rbase + t) = S::pack(yo);
            } else {
#pragma unroll
                for (int i = 0; i < VW; ++i)
                    if (row_ok && t + i < t_end) IO::store(y, rbase + t + i, yo[i]);
            }
        }
        __syncthreads();
    }

    if (FULL) {
        // the sequence that is current at the chunk end ends with it
        if (sp.end == t_end) store_final_state<4>(a, sp.s, d, lane_ok, 4 * q, h);
        // empty packed sequences keep their initial state
        if (EXT && a.cu && a.last_state && j == 0) {
            for (int64_t s = 0; s < a.n_seqs; ++s) {
                if (cu_at(a, s) != cu_at(a, s + 1)) continue;
                load_start_state<4>(a, s, dcl, lane_ok, 4 * q, h);
                store_final_state<4>(a, s, d, lane_ok, 4 * q, h);
            }
        }
    } else {
        dt_sum_out = dt_sum;
    }
}

// One chunk per wavefront: the aggregate pass (FULL = false, chunks
// 0 .. J-2, into the workspace) or the pass that writes y, of the two-pass
// schedule (the chunk start states come from h_start or the fold).
template <class IO, bool FULL, bool VEC, bool EXT, bool ZOH>
__global__ __launch_bounds__(64) void quad_kernel(ScanArgs a) {
    using Q = QuadTile<IO, FULL>;
    __shared__ __attribute__((aligned(16))) float s_dt[Q::n_dt];
    __shared__ __attribute__((aligned(16))) float s_w[Q::n_w];
    __shared__ __attribute__((aligned(16))) float s_du[Q::n_du];
    __shared__ __attribute__((aligned(16))) float s_B[Q::n_B];
    __shared__ __attribute__((aligned(16))) float s_C[Q::n_C];
    const int64_t j = blockIdx.y;
    float h[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float dt_sum = 0.0f, keep = 0.0f;
    quad_pass<IO, FULL, VEC, EXT, ZOH, false, true>(a, blockIdx.x, j, j * a.K, chunk_end(a, j), h,
                                                    dt_sum, keep, s_dt, s_w, s_du, s_B, s_C);
    if (!FULL) {
        const int lane = threadIdx.x;
        const int q = lane >> 4;
        const int64_t b = blockIdx.x / a.n_cblk;
        const int64_t d = static_cast<int64_t>(blockIdx.x % a.n_cblk) * 16 + (lane & 15);
        if (lane == 0 && blockIdx.x % a.n_cblk == 0) a.keep[b * a.J + j] = keep;
        if (d >= a.D) return;
        const size_t cd = (static_cast<size_t>(b) * a.D + d) * a.J + j;
        *reinterpret_cast<float4 *>(a.hend + cd * 16 + 4 * q) = make_float4(h[0], h[1], h[2], h[3]);
        if (q == 0) a.dtsum[cd] = dt_sum;
    }
}

// The whole chunked scan in one launch (up to kFoldMaxChunks chunks): the
// wavefront of chunk j
//  1. runs the aggregate pass of its own chunk (unless it is the last) and
//     publishes the result: the end state and sum of dt in the workspace,
//     then this launch's epoch in its flag;
//  2. waits until the chunks 0 .. j-1 of its 16-channel block have
//     published, and folds their transfer operators, in chunk order, into
//     its start state [ufo.work, "Accelerating state-space models ...",
//     §3.1: chunk operators combined, start states broadcast];
//  3. runs the pass that writes y from that state.
// Scheduling: a SIMD issues from its oldest wavefront first, so without
// help the first chunk on each SIMD would run its y pass while the later
// chunks' aggregate passes and folds, which the y passes wait for, starve.
// Steps 1 and 2 therefore run at raised wave priority (s_setprio), step 3 at
// the default.
// Bounded waiting: the wait ends at a real-time deadline (a.spin_ticks of
// the 100 MHz clock); after it the wavefront computes each missing
// aggregate itself, with the same code and so the same bits, and never
// depends on another wavefront being scheduled.  spin_ticks = 0 makes every
// chunk independent: nothing is published or awaited, each chunk computes
// all operators before it.
// Memory ordering across the XCDs' separate L2 caches: the operators and
// the flag are written with agent-scope atomic stores (sc1: written through
// to the device-coherent level) and the flag only after s_waitcnt has seen
// the operator stores complete; readers load flag and operators with
// agent-scope atomic loads (sc1: read from the coherent level, never a
// stale L2 line), the operators only after the flag load has returned.  A
// release/acquire fence pair would instead write back and invalidate whole
// L2 caches per wavefront (measured: 2.7x slower on the Mamba-130M layer).
// Flags hold a 64-bit epoch that is new for every launch, so the workspace
// needs no clearing between launches (graph capture clears it, see the
// launch).
// Wait until this wavefront's stores have completed, before the flag store
// that announces them.  s_waitcnt alone is not a memory operation to the
// compiler, so compiler-only fences on both sides keep the operator stores
// before it and the flag store after it (no cache write-back is emitted).
__device__ __forceinline__ void publish_wait() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <class IO, bool VEC, bool EXT, bool ZOH>
__global__ __launch_bounds__(64) void quad_fused_kernel(ScanArgs a) {
    using Q = QuadTile<IO, true>;
    __shared__ __attribute__((aligned(16))) float s_dt[Q::n_dt];
    __shared__ __attribute__((aligned(16))) float s_w[Q::n_w];
    __shared__ __attribute__((aligned(16))) float s_du[Q::n_du];
    __shared__ __attribute__((aligned(16))) float s_B[Q::n_B];
    __shared__ __attribute__((aligned(16))) float s_C[Q::n_C];
    const int lane = threadIdx.x;
    const int q = lane >> 4;
    const int64_t j = blockIdx.y;
    const int64_t b = blockIdx.x / a.n_cblk;
    const int64_t d = static_cast<int64_t>(blockIdx.x % a.n_cblk) * 16 + (lane & 15);
    const bool lane_ok = d < a.D;
    const int64_t dcl = lane_ok ? d : a.D - 1;
    const size_t cd0 = (static_cast<size_t>(b) * a.D + dcl) * a.J;
    uint64_t *flags = a.flags + static_cast<size_t>(blockIdx.x) * a.J;
    float h[4], dt_sum = 0.0f, keep = 0.0f;
    constexpr int kAgent = __HIP_MEMORY_SCOPE_AGENT;

    // 1. this chunk's operator, for the chunks after it (no one reads it
    // when chunks do not wait)
    __builtin_amdgcn_s_setprio(3);
    if (j + 1 < a.J && a.spin_ticks != 0) {
        quad_pass<IO, false, VEC, EXT, ZOH, false>(a, blockIdx.x, j, j * a.K, chunk_end(a, j), h,
                                                   dt_sum, keep, s_dt, s_w, s_du, s_B, s_C);
        if (lane_ok) {
            float *he = a.hend + (cd0 + j) * 16 + 4 * q;
#pragma unroll
            for (int k = 0; k < 4; ++k) __hip_atomic_store(he + k, h[k], __ATOMIC_RELAXED, kAgent);
            if (q == 0) __hip_atomic_store(a.dtsum + cd0 + j, dt_sum, __ATOMIC_RELAXED, kAgent);
        }
        publish_wait();   // the operator stores are complete
        if (lane == 0) __hip_atomic_store(flags + j, a.epoch, __ATOMIC_RELAXED, kAgent);
    }

    // 2. the start state: fold the operators of chunks 0 .. j-1 (a chunk at
    // which a sequence starts loads its own start state in the pass)
    h[0] = h[1] = h[2] = h[3] = 0.0f;
    if (j > 0 && !seq_pos<EXT>(a, b, j * a.K).reset) {
        // lane i < j watches chunk i's flag
        uint64_t ready = 0;
        const uint64_t deadline = __builtin_amdgcn_s_memrealtime() + a.spin_ticks;
        while (a.spin_ticks != 0) {
            const bool mine =
                lane >= j || __hip_atomic_load(flags + lane, __ATOMIC_RELAXED, kAgent) == a.epoch;
            ready = __ballot(mine);
            if (ready == ~0ull || __builtin_amdgcn_s_memrealtime() >= deadline) break;
            __builtin_amdgcn_s_sleep(2);
        }
        float A2[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int n = 4 * q + k;
            const float v = a.A[dcl * a.N + (n < a.N ? n : a.N - 1)];
            A2[k] = (lane_ok && n < a.N) ? v * kLog2e : 0.0f;
        }
        if (ready != ~0ull) {
            // operators not published in time: compute them here and write
            // them to their slots (the same bits their owner writes, if it
            // ever does)
            for (int64_t i = 0; i < j; ++i) {
                if ((ready >> i) & 1) continue;
                float e[4], sdt, kp;
                quad_pass<IO, false, VEC, EXT, ZOH, false>(a, blockIdx.x, i, i * a.K,
                                                           chunk_end(a, i), e, sdt, kp, s_dt, s_w,
                                                           s_du, s_B, s_C);
                if (lane_ok) {
                    float *he = a.hend + (cd0 + i) * 16 + 4 * q;
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        __hip_atomic_store(he + k, e[k], __ATOMIC_RELAXED, kAgent);
                    if (q == 0) __hip_atomic_store(a.dtsum + cd0 + i, sdt, __ATOMIC_RELAXED, kAgent);
                }
            }
            publish_wait();
        }
        // 8 operators at a time: their loads are issued together
        constexpr int kBatch = 8;
        for (int64_t i0 = 0; i0 < j; i0 += kBatch) {
            float e[kBatch][4], sdt[kBatch];
#pragma unroll
            for (int m = 0; m < kBatch; ++m) {
                const int64_t i = i0 + m < j ? i0 + m : j - 1;
                const float *he = a.hend + (cd0 + i) * 16 + 4 * q;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    e[m][k] = __hip_atomic_load(he + k, __ATOMIC_RELAXED, kAgent);
                sdt[m] = __hip_atomic_load(a.dtsum + cd0 + i, __ATOMIC_RELAXED, kAgent);
            }
#pragma unroll
            for (int m = 0; m < kBatch; ++m) {
                const int64_t i = i0 + m;
                if (i < j) {
                    const int64_t tb = i * a.K;
                    const int64_t te = tb + a.K < a.L ? tb + a.K : a.L;
                    const SeqPos sp = seq_pos<EXT>(a, b, tb);
                    const bool kept = !sp.reset && sp.end >= te;
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        h[k] = __builtin_fmaf(kept ? exp2_hw(A2[k] * sdt[m]) : 0.0f, h[k],
                                              e[m][k]);
                }
            }
        }
    }

    // 3. y and the final states
    __builtin_amdgcn_s_setprio(0);
    quad_pass<IO, true, VEC, EXT, ZOH, true>(a, blockIdx.x, j, j * a.K, chunk_end(a, j), h,
                                             dt_sum, keep, s_dt, s_w, s_du, s_B, s_C);
}

// Serial walks balanced over the SIMDs (d_state <= 16, no packed sequences,
// convolution or ZOH).  When the 16-channel blocks number, say, 2.5 per SIMD,
// one wavefront per block leaves half the SIMDs with a third whole sequence
// to scan and the other half idle for that long.  Here the first n_full
// blocks (a whole number of rounds) each walk the whole sequence, and each
// block after them is cut into two chunks on two wavefronts, which take the
// next slot on every SIMD:
//   chunk 0 (tokens 0 .. K-1): the aggregate pass of its tokens at raised
//     wave priority, published with this launch's epoch (as the one-launch
//     kernel does), then its y pass;
//   chunk 1 (tokens K .. L-1): waits for chunk 0's end state (bounded; past
//     the deadline it computes it itself), then its y pass from it.
// K is chosen so that both chunks cost about the same (chunk 0 scans its
// tokens twice).  Workspace: the J = 2 layout of the chunked plans.
template <class IO, bool VEC>
__global__ __launch_bounds__(64, 3) void quad_split_kernel(ScanArgs a) {
    using Q = QuadTile<IO, true>;
    __shared__ __attribute__((aligned(16))) float s_dt[Q::n_dt];
    __shared__ __attribute__((aligned(16))) float s_w[Q::n_w];
    __shared__ __attribute__((aligned(16))) float s_du[Q::n_du];
    __shared__ __attribute__((aligned(16))) float s_B[Q::n_B];
    __shared__ __attribute__((aligned(16))) float s_C[Q::n_C];
    constexpr int kAgent = __HIP_MEMORY_SCOPE_AGENT;
    const int64_t w = blockIdx.x;
    float h[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float dt_sum = 0.0f, keep = 0.0f;
    if (w < a.n_full) {
        quad_pass<IO, true, VEC, false, false, false, true>(a, w, 0, 0, a.L, h, dt_sum, keep, s_dt,
                                                            s_w, s_du, s_B, s_C);
        return;
    }
    const int64_t blk = a.n_full + (w - a.n_full) / 2;
    const int64_t j = (w - a.n_full) % 2;
    const int lane = threadIdx.x;
    const int q = lane >> 4;
    const int64_t b = blk / a.n_cblk;
    const int64_t d = static_cast<int64_t>(blk % a.n_cblk) * 16 + (lane & 15);
    const bool lane_ok = d < a.D;
    const int64_t dcl = lane_ok ? d : a.D - 1;
    const size_t cd0 = (static_cast<size_t>(b) * a.D + dcl) * 2;
    uint64_t *flag = a.flags + static_cast<size_t>(blk) * 2;
    float *he = a.hend + cd0 * 16 + 4 * q;
    if (j == 0) {
        // chunk 0's end state (from the start state), for chunk 1
        if (a.spin_ticks != 0) {
            __builtin_amdgcn_s_setprio(3);
            quad_pass<IO, false, VEC, false, false, false>(a, blk, 0, 0, a.K, h, dt_sum, keep,
                                                           s_dt, s_w, s_du, s_B, s_C);
            if (lane_ok) {
#pragma unroll
                for (int k = 0; k < 4; ++k) __hip_atomic_store(he + k, h[k], __ATOMIC_RELAXED, kAgent);
            }
            publish_wait();   // the end state is stored
            if (lane == 0) __hip_atomic_store(flag, a.epoch, __ATOMIC_RELAXED, kAgent);
        }
        quad_pass<IO, true, VEC, false, false, false, true>(a, blk, 0, 0, a.K, h, dt_sum, keep,
                                                            s_dt, s_w, s_du, s_B, s_C);
        return;
    }
    // chunk 1: chunk 0 begins the sequence, so the state entering chunk 1 is
    // chunk 0's end state itself
    bool ready = false;
    const uint64_t deadline = __builtin_amdgcn_s_memrealtime() + a.spin_ticks;
    while (a.spin_ticks != 0) {
        ready = __ballot(lane == 0 && __hip_atomic_load(flag, __ATOMIC_RELAXED, kAgent) == a.epoch) != 0;
        if (ready || __builtin_amdgcn_s_memrealtime() >= deadline) break;
        __builtin_amdgcn_s_sleep(2);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the end-state loads stay after the flag's
    if (ready) {
#pragma unroll
        for (int k = 0; k < 4; ++k) h[k] = __hip_atomic_load(he + k, __ATOMIC_RELAXED, kAgent);
    } else {
        // not published in time: compute it here (the same bits)
        quad_pass<IO, false, VEC, false, false, false>(a, blk, 0, 0, a.K, h, dt_sum, keep, s_dt,
                                                       s_w, s_du, s_B, s_C);
    }
    quad_pass<IO, true, VEC, false, false, true, true>(a, blk, 1, a.K, a.L, h, dt_sum, keep, s_dt,
                                                       s_w, s_du, s_B, s_C);
}

// ============================================================ group kernel (N > 16)
// The path for 16 < d_state <= 256: the state dimension is split into groups
// of 32 states on G wavefronts of one workgroup (the state-dimension groups
// of the ufo.work article, §3.2), all serving the same 16 channels.  In
// wavefront g, lane l serves channel c = l % 16 and the 8 states
// 32g + 8q .. 32g + 8q + 7, q = l / 16, in VGPRs.
//
// Tile: 16 channels x 16 tokens.  Per tile:
//  (a) the workgroup loads and converts the tile's u, delta, z (one to four
//      consecutive tokens per thread) into dt, w = dt u, D u and silu(z) rows
//      in LDS, and the tile's B and C rows (state-major, two 4-token pieces of
//      each per thread, states n >= N zeroed); the next tile's values are
//      loaded meanwhile;
//  (b) every wavefront walks the tile 4 tokens at a time: ds_read_b128 gives
//      4 tokens of dt, of w and of B[32g + 8q + (lane % 8)], which enters
//      w B through the DPP operand row_newbcast:k; C for 4 tokens is one
//      ds_read_b128 per state.  The 4 lane-rows' partial C.h are summed with
//      the same permlane butterfly as the quad kernel, and each wavefront
//      writes its group's partial y to LDS;
//  (c) the partials of the G groups are added in group order (a fixed order:
//      the result does not depend on timing), then + D u, times silu(z),
//      and stored.
#ifndef SSM_GROUP_WAVES_PER_SIMD
#define SSM_GROUP_WAVES_PER_SIMD 4
#endif
template <class IO, int G, bool FULL, bool VEC, bool EXT, bool ZOH>
__global__ __launch_bounds__(64 * G, SSM_GROUP_WAVES_PER_SIMD) void group_kernel(ScanArgs a) {
    using IT = typename IO::T;
    using P = Piece4<IO>;
    constexpr int T = 16;                           // tokens per tile
    constexpr int TP = T + 4;                       // padded LDS row
    constexpr int QC = 16;                          // channels per workgroup
    constexpr int NS = 32 * G;                      // padded states per channel
    constexpr int NT = 64 * G;                      // threads
    constexpr int EPT = G >= 4 ? 1 : 4 / G;         // u/delta/z elements per thread
    constexpr int NACT = QC * T / EPT;              // threads that hold elements
    static_assert(NACT <= NT, "element mapping");
    __shared__ __attribute__((aligned(16))) float s_dt[QC * TP];
    // rows start 4 floats in: the 4 floats before a row (the previous row's
    // padding) keep the convolution inputs of the 4 tokens before the tile
    __shared__ __attribute__((aligned(16))) float s_w[QC * TP + 4];
    __shared__ __attribute__((aligned(16))) float s_du[FULL ? QC * TP : 4];
    __shared__ __attribute__((aligned(16))) float s_g[FULL ? QC * TP : 4];
    __shared__ __attribute__((aligned(16))) float s_B[NS * TP];
    __shared__ __attribute__((aligned(16))) float s_C[FULL ? NS * TP : 4];
    __shared__ __attribute__((aligned(16))) float s_yp[FULL ? G * QC * TP : 4];

    const IT *__restrict__ u = static_cast<const IT *>(a.u);
    const IT *__restrict__ dl = static_cast<const IT *>(a.delta);
    const IT *__restrict__ z = static_cast<const IT *>(a.z);
    const IT *__restrict__ Bm = static_cast<const IT *>(a.B);
    const IT *__restrict__ Cm = static_cast<const IT *>(a.C);
    IT *__restrict__ y = static_cast<IT *>(a.y);

    const int tid = threadIdx.x;
    const int g = tid >> 6;                         // state group of this wavefront
    const int lane = tid & 63;
    const int c = lane & 15;
    const int q = lane >> 4;
    const int64_t b = blockIdx.x / a.n_cblk;
    const int64_t j = blockIdx.y;
    const int64_t d0 = static_cast<int64_t>(blockIdx.x % a.n_cblk) * QC;
    const int64_t d = d0 + c;
    const bool lane_ok = d < a.D;
    const int64_t L = a.L;
    const int64_t t_begin = j * a.K;
    const int64_t t_end = t_begin + a.K < L ? t_begin + a.K : L;
    const bool gate = a.z != nullptr;

    // ---- element mapping for u, delta, z, y: row er, tokens [et, et + EPT)
    const bool act = tid < NACT;
    const int er = (tid * EPT) >> 4;
    const int et = (tid * EPT) & 15;
    const int64_t edr = d0 + (act ? er : 0);
    const bool erow_ok = act && edr < a.D;
    const size_t ebase = (static_cast<size_t>(b) * a.D + (edr < a.D ? edr : a.D - 1)) * L;
    const float ebias = (erow_ok && a.delta_bias) ? a.delta_bias[edr] : 0.0f;
    const float eD = (erow_ok && a.Dskip) ? a.Dskip[edr] : 0.0f;
    const int64_t edrc = edr < a.D ? edr : a.D - 1;
    const bool conv = EXT && a.conv_w > 0;                 // u holds the convolution's input
    const float4 cw = (conv && act) ? conv_taps(a, edrc) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float cbias = (conv && act && a.conv_bias) ? a.conv_bias[edrc] : 0.0f;

    // ---- B/C piece mapping: pieces tid and tid + NT of each tensor;
    // piece p = row p / 4 (a state), tokens 4 (p % 4) .. + 3
    const int pr0 = tid >> 2, pr1 = (tid + NT) >> 2;
    const int ps = (tid & 3) * 4;                   // same column for both (NT % 4 == 0)
    const bool pok0 = pr0 < a.N, pok1 = pr1 < a.N;
    const size_t pb0 = (static_cast<size_t>(b) * a.N + (pok0 ? pr0 : a.N - 1)) * L;
    const size_t pb1 = (static_cast<size_t>(b) * a.N + (pok1 ? pr1 : a.N - 1)) * L;

    // prefetch registers (named; no arrays carried around the loop)
    float eu0 = 0.f, eu1 = 0.f, eu2 = 0.f, eu3 = 0.f;
    float ed0 = 0.f, ed1 = 0.f, ed2 = 0.f, ed3 = 0.f;
    float ez0 = 0.f, ez1 = 0.f, ez2 = 0.f, ez3 = 0.f;
    typename P::V vb0{}, vb1{}, vc0{}, vc1{};
    auto eload = [&](const IT *p, int64_t t, int i) {
        const int64_t tt = t + i < t_end ? t + i : t_end - 1;
        return IO::load(p, ebase + tt);
    };
    auto pload = [&](const IT *p, size_t base, int64_t t) {
        if (VEC) {
            const int64_t tc = t < t_end ? t : t_end - 4;   // t_end >= 4 here
            return *reinterpret_cast<const typename P::V *>(p + base + tc);
        }
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t tt = t + i < t_end ? t + i : t_end - 1;
            e[i] = IO::load(p, base + tt);
        }
        return P::pack(e);
    };
    auto load_tile = [&](int64_t t0) {
        if (act) {
            const int64_t t = t0 + et;
            eu0 = eload(u, t, 0); ed0 = eload(dl, t, 0);
            if (EPT > 1) { eu1 = eload(u, t, 1); ed1 = eload(dl, t, 1); }
            if (EPT > 2) {
                eu2 = eload(u, t, 2); ed2 = eload(dl, t, 2);
                eu3 = eload(u, t, 3); ed3 = eload(dl, t, 3);
            }
            if (FULL && gate) {
                ez0 = eload(z, t, 0);
                if (EPT > 1) ez1 = eload(z, t, 1);
                if (EPT > 2) { ez2 = eload(z, t, 2); ez3 = eload(z, t, 3); }
            }
        }
        vb0 = pload(Bm, pb0, t0 + ps);
        vb1 = pload(Bm, pb1, t0 + ps);
        if (FULL) {
            vc0 = pload(Cm, pb0, t0 + ps);
            vc1 = pload(Cm, pb1, t0 + ps);
        }
    };

    // ---- per-lane constants and initial state: states n = 32g + 8q + k
    const int64_t dcl = lane_ok ? d : a.D - 1;
    const int nb = 32 * g + 8 * q;
    float A2[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int n = nb + k;
        const float v = a.A[dcl * a.N + (n < a.N ? n : a.N - 1)];
        A2[k] = (lane_ok && n < a.N) ? v * kLog2e : 0.0f;
    }
    float h[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) h[k] = 0.0f;
    const size_t cd0 = (static_cast<size_t>(b) * a.D + dcl) * a.J;
    const size_t cd = cd0 + j;
    SeqPos sp = seq_pos<EXT>(a, b, t_begin);
    const float keep = (!sp.reset && sp.end >= t_end) ? 1.0f : 0.0f;
    load_tile(t_begin);
    if (sp.reset) {
        load_start_state<8>(a, sp.s, dcl, lane_ok, nb, h);
    } else if (FULL) {
        if (a.hstart) {
            const float4 v0 = *reinterpret_cast<const float4 *>(a.hstart + cd * NS + nb);
            const float4 v1 = *reinterpret_cast<const float4 *>(a.hstart + cd * NS + nb + 4);
            h[0] = v0.x; h[1] = v0.y; h[2] = v0.z; h[3] = v0.w;
            h[4] = v1.x; h[5] = v1.y; h[6] = v1.z; h[7] = v1.w;
        } else {
            for (int64_t i = 0; i < j; ++i) {
                const float sdt = a.dtsum[cd0 + i];
                const float4 v0 = *reinterpret_cast<const float4 *>(a.hend + (cd0 + i) * NS + nb);
                const float4 v1 = *reinterpret_cast<const float4 *>(a.hend + (cd0 + i) * NS + nb + 4);
                const float he[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    h[k] = __builtin_fmaf(chunk_decay(a, b, i, A2[k], sdt), h[k], he[k]);
            }
        }
        if (!lane_ok) {
#pragma unroll
            for (int k = 0; k < 8; ++k) h[k] = 0.0f;
        }
    }
    float dt_sum = 0.0f;
    if (conv && act && et == 0) {
        // convolution inputs of the 4 tokens before the chunk
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t tt = t_begin - 4 + k;
            s_w[er * TP + k] = tt >= 0 ? IO::load(u, ebase + tt) : 0.0f;
        }
    }

    const int64_t n_tiles = (t_end - t_begin + T - 1) / T;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += T) {
        fair_prio((t0 - t_begin) / T, n_tiles);
        float uc[EPT];
        if (conv) {
            // (a0) the scan input u = act(conv(x)) of this thread's elements
            const float xr[4] = {eu0, eu1, eu2, eu3};
            const int o = er * TP + et;
            if (act) {
#pragma unroll
                for (int i = 0; i < EPT; ++i) s_w[4 + o + i] = xr[i];
            }
            __syncthreads();
            if (act) {
                const int64_t st_cur = (EXT && a.cu) ? cu_at(a, sp.s) : 0;
                conv_run<EPT, EXT>(a, &s_w[4 + o], t0 + et, sp, st_cur, edrc, cw, cbias, uc);
            }
            __syncthreads();
            if (act) {
                // keep the tile's last 4 inputs for the next tile
#pragma unroll
                for (int i = 0; i < EPT; ++i)
                    if (et + i >= T - 4) s_w[er * TP + et + i - (T - 4)] = xr[i];
                if (FULL && a.u_out) {
#pragma unroll
                    for (int i = 0; i < EPT; ++i) {
                        const int64_t t = t0 + et + i;
                        if (erow_ok && t < t_end) IO::store(static_cast<IT *>(a.u_out), ebase + t, uc[i]);
                    }
                }
            }
        }
        // (a) convert and stage the tile
        if (act) {
            const float xu[4] = {conv ? uc[0] : eu0, conv && EPT > 1 ? uc[EPT > 1 ? 1 : 0] : eu1,
                                 conv && EPT > 2 ? uc[EPT > 2 ? 2 : 0] : eu2,
                                 conv && EPT > 3 ? uc[EPT > 3 ? 3 : 0] : eu3};
            const float xd[4] = {ed0, ed1, ed2, ed3};
            const float xz[4] = {ez0, ez1, ez2, ez3};
            const int o = er * TP + et;
#pragma unroll
            for (int i = 0; i < EPT; ++i) {
                const bool ok = erow_ok && t0 + et + i < t_end;
                const float x = xd[i] + ebias;
                const float dt = ok ? (a.softplus ? softplus_f32(x) : x) : 0.0f;
                const float uu = ok ? xu[i] : 0.0f;
                s_dt[o + i] = dt;
                s_w[4 + o + i] = dt * uu;
                if (FULL) {
                    s_du[o + i] = eD * uu;
                    s_g[o + i] = (FULL && gate) ? silu_f32(ok ? xz[i] : 0.0f) : 1.0f;
                }
            }
        }
        {
            float e[4];
            P::unpack(vb0, e);
            *reinterpret_cast<float4 *>(&s_B[pr0 * TP + ps]) =
                pok0 ? make_float4(e[0], e[1], e[2], e[3]) : make_float4(0.f, 0.f, 0.f, 0.f);
            P::unpack(vb1, e);
            *reinterpret_cast<float4 *>(&s_B[pr1 * TP + ps]) =
                pok1 ? make_float4(e[0], e[1], e[2], e[3]) : make_float4(0.f, 0.f, 0.f, 0.f);
            if (FULL) {
                P::unpack(vc0, e);
                *reinterpret_cast<float4 *>(&s_C[pr0 * TP + ps]) =
                    pok0 ? make_float4(e[0], e[1], e[2], e[3]) : make_float4(0.f, 0.f, 0.f, 0.f);
                P::unpack(vc1, e);
                *reinterpret_cast<float4 *>(&s_C[pr1 * TP + ps]) =
                    pok1 ? make_float4(e[0], e[1], e[2], e[3]) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        load_tile(t0 + T);
        __syncthreads();

        // (b) the recurrence of this wavefront's 32 states
        const int rowc = c * TP;
        const int brow = (nb + (lane & 7)) * TP;
        const int crow = nb * TP;
        if (EXT && sp.end < t0 + T && sp.end < t_end) {
            // a sequence boundary inside the tile: token by token
            for (int k = 0; k < T; ++k) {
                const int64_t t = t0 + k;
                if (t == sp.end && t < t_end) {
                    if (FULL) store_final_state<8>(a, sp.s, d, lane_ok, nb, h);
                    sp = seq_pos<EXT>(a, b, t);
                    load_start_state<8>(a, sp.s, dcl, lane_ok, nb, h);
                }
                const float dt = s_dt[rowc + k], w = s_w[4 + rowc + k], Bk = s_B[brow + k];
                h[0] = state_step<ZOH>(dt, A2[0], h[0], row_bcast<0>(Bk) * w);
                h[1] = state_step<ZOH>(dt, A2[1], h[1], row_bcast<1>(Bk) * w);
                h[2] = state_step<ZOH>(dt, A2[2], h[2], row_bcast<2>(Bk) * w);
                h[3] = state_step<ZOH>(dt, A2[3], h[3], row_bcast<3>(Bk) * w);
                h[4] = state_step<ZOH>(dt, A2[4], h[4], row_bcast<4>(Bk) * w);
                h[5] = state_step<ZOH>(dt, A2[5], h[5], row_bcast<5>(Bk) * w);
                h[6] = state_step<ZOH>(dt, A2[6], h[6], row_bcast<6>(Bk) * w);
                h[7] = state_step<ZOH>(dt, A2[7], h[7], row_bcast<7>(Bk) * w);
                if (FULL) {
                    float acc = s_C[crow + k] * h[0];
#pragma unroll
                    for (int i = 1; i < 8; ++i) acc = __builtin_fmaf(s_C[crow + i * TP + k], h[i], acc);
                    acc += __shfl_xor(acc, 16);
                    acc += __shfl_xor(acc, 32);
                    if (q == 0) s_yp[g * QC * TP + rowc + k] = acc;
                } else {
                    dt_sum += dt;
                }
            }
        } else {
#pragma unroll
        for (int c4 = 0; c4 < T; c4 += 4) {
            const float4 dt4 = *reinterpret_cast<const float4 *>(&s_dt[rowc + c4]);
            const float4 w4 = *reinterpret_cast<const float4 *>(&s_w[4 + rowc + c4]);
            const float4 B4 = *reinterpret_cast<const float4 *>(&s_B[brow + c4]);
            float4 Cq[8];
            if (FULL) {
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    Cq[k] = *reinterpret_cast<const float4 *>(&s_C[crow + k * TP + c4]);
            }
            const float dtv[4] = {dt4.x, dt4.y, dt4.z, dt4.w};
            const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
            const float bv[4] = {B4.x, B4.y, B4.z, B4.w};
            float accv[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float dt = dtv[k], w = wv[k], Bk = bv[k];
                h[0] = state_step<ZOH>(dt, A2[0], h[0], row_bcast<0>(Bk) * w);
                h[1] = state_step<ZOH>(dt, A2[1], h[1], row_bcast<1>(Bk) * w);
                h[2] = state_step<ZOH>(dt, A2[2], h[2], row_bcast<2>(Bk) * w);
                h[3] = state_step<ZOH>(dt, A2[3], h[3], row_bcast<3>(Bk) * w);
                h[4] = state_step<ZOH>(dt, A2[4], h[4], row_bcast<4>(Bk) * w);
                h[5] = state_step<ZOH>(dt, A2[5], h[5], row_bcast<5>(Bk) * w);
                h[6] = state_step<ZOH>(dt, A2[6], h[6], row_bcast<6>(Bk) * w);
                h[7] = state_step<ZOH>(dt, A2[7], h[7], row_bcast<7>(Bk) * w);
                if (FULL) {
                    const float ck[8] = {
                        k == 0 ? Cq[0].x : k == 1 ? Cq[0].y : k == 2 ? Cq[0].z : Cq[0].w,
                        k == 0 ? Cq[1].x : k == 1 ? Cq[1].y : k == 2 ? Cq[1].z : Cq[1].w,
                        k == 0 ? Cq[2].x : k == 1 ? Cq[2].y : k == 2 ? Cq[2].z : Cq[2].w,
                        k == 0 ? Cq[3].x : k == 1 ? Cq[3].y : k == 2 ? Cq[3].z : Cq[3].w,
                        k == 0 ? Cq[4].x : k == 1 ? Cq[4].y : k == 2 ? Cq[4].z : Cq[4].w,
                        k == 0 ? Cq[5].x : k == 1 ? Cq[5].y : k == 2 ? Cq[5].z : Cq[5].w,
                        k == 0 ? Cq[6].x : k == 1 ? Cq[6].y : k == 2 ? Cq[6].z : Cq[6].w,
                        k == 0 ? Cq[7].x : k == 1 ? Cq[7].y : k == 2 ? Cq[7].z : Cq[7].w};
                    float s0 = ck[0] * h[0];
                    float s1 = ck[1] * h[1];
                    s0 = __builtin_fmaf(ck[2], h[2], s0);
                    s1 = __builtin_fmaf(ck[3], h[3], s1);
                    s0 = __builtin_fmaf(ck[4], h[4], s0);
                    s1 = __builtin_fmaf(ck[5], h[5], s1);
                    s0 = __builtin_fmaf(ck[6], h[6], s0);
                    s1 = __builtin_fmaf(ck[7], h[7], s1);
                    accv[k] = s0 + s1;
                } else {
                    dt_sum += dt;
                }
            }
            if (FULL) {
                const auto s01 = __builtin_amdgcn_permlane16_swap(
                    __float_as_uint(accv[0]), __float_as_uint(accv[1]), false, false);
                const auto s23 = __builtin_amdgcn_permlane16_swap(
                    __float_as_uint(accv[2]), __float_as_uint(accv[3]), false, false);
                const float p01 = __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
                const float p23 = __uint_as_float(s23[0]) + __uint_as_float(s23[1]);
                const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(p01),
                                                                __float_as_uint(p23), false, false);
                s_yp[g * QC * TP + rowc + c4 + q] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
            }
        }
        }

        // (c) sum the groups' partials in group order, finish and store y
        if (FULL) {
            __syncthreads();
            if (act) {
                const int o = er * TP + et;
#pragma unroll
                for (int i = 0; i < EPT; ++i) {
                    float acc = s_yp[o + i];
#pragma unroll
                    for (int gg = 1; gg < G; ++gg) acc += s_yp[gg * QC * TP + o + i];
                    const float v = (acc + s_du[o + i]) * s_g[o + i];
                    const int64_t t = t0 + et + i;
                    if (erow_ok && t < t_end) IO::store(y, ebase + t, v);
                }
            }
        }
        __syncthreads();
    }

    if (FULL) {
        if (sp.end == t_end) store_final_state<8>(a, sp.s, d, lane_ok, nb, h);
        if (EXT && a.cu && a.last_state && j == 0) {
            for (int64_t s = 0; s < a.n_seqs; ++s) {
                if (cu_at(a, s) != cu_at(a, s + 1)) continue;
                load_start_state<8>(a, s, dcl, lane_ok, nb, h);
                store_final_state<8>(a, s, d, lane_ok, nb, h);
            }
        }
    } else {
        if (tid == 0 && blockIdx.x % a.n_cblk == 0) a.keep[b * a.J + j] = keep;
        if (!lane_ok) return;
        float *he = a.hend + cd * NS + nb;
        *reinterpret_cast<float4 *>(he) = make_float4(h[0], h[1], h[2], h[3]);
        *reinterpret_cast<float4 *>(he + 4) = make_float4(h[4], h[5], h[6], h[7]);
        if (g == 0 && q == 0) a.dtsum[cd] = dt_sum;
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
        const float v = a.A[d * a.N + (n < a.N ? n : a.N - 1)];
        A2[i] = n < a.N ? v * kLog2e : 0.0f;
        hin[i] = 0.0f;
    }
    for (int64_t j0 = 0; j0 < a.J; j0 += kWave) {
        const int64_t jj = j0 + lane;
        const bool ok = jj < a.J;                    // h_start is written for every chunk
        const bool has_op = jj < a.J - 1;            // the last chunk acts as identity
        const size_t cd = static_cast<size_t>(bd) * a.J + (ok ? jj : 0);
        // cd is a valid index for every lane; the last chunk's slots hold no
        // operator, so their (finite or not) contents are replaced by select.
        const float sdt_raw = a.dtsum[cd];
        const float sdt = has_op ? sdt_raw : 0.0f;
        // a chunk in which a sequence starts forgets its incoming state
        const bool kept = a.keep[(bd / a.D) * a.J + (ok ? jj : 0)] != 0.0f;
        const float *he = a.hend + cd * Npad + g * kGroup;
        float *hs = a.hstart + cd * Npad + g * kGroup;
        float hev[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) hev[i] = he[i];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            float av = has_op ? (kept ? exp2_hw(A2[i] * sdt) : 0.0f) : 1.0f;
            float bv = has_op ? hev[i] : 0.0f;
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
// Profiling events (optional, both or neither): the scan's first dispatch
// records ev_begin at its start and its last dispatch ev_end at its end
// (hipExtLaunchKernelGGL), so that their interval covers every pass of the
// scan -- aggregate pass, carry kernel and the pass that writes y -- as a
// profiler's kernel trace measures them, without event packets in the queue.
struct Dispatch {
    hipEvent_t begin = nullptr, end = nullptr;
    hipStream_t s = nullptr;
    Dispatch(const ScanArgs &a, hipStream_t st) : s(st) {
        if (a.ev_begin && a.ev_end) { begin = a.ev_begin; end = a.ev_end; }
    }
    template <class Kern, class... Args>
    void operator()(bool last, Kern kernel, dim3 grid, dim3 block, Args... args) {
        if (begin || (last && end)) {
            hipExtLaunchKernelGGL(kernel, grid, block, 0, s, begin, last ? end : nullptr, 0,
                                  args...);
            begin = nullptr;
        } else {
            hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
        }
    }
};

// The vector path of the serial walks (quad_pass) reaches a block's 16 rows,
// and a batch row's N rows of B and C, through buffer views of under 2^31
// bytes: its offsets reach 16 L elements plus two tiles, and the checkpoint
// view's 16 rows of n_ck 64-byte entries.
template <class IO>
static bool quad_views_fit(const ScanArgs &a) {
    const uint64_t e = (16 * static_cast<uint64_t>(a.L) + 64) * sizeof(typename IO::T);
    const uint64_t c = a.ckpt ? 16 * static_cast<uint64_t>(a.n_ck) * 64 : 0;
    return e < (1ull << 31) && c < (1ull << 31);
}

template <class IO, bool VEC, bool EXT, bool ZOH>
static hipError_t launch_quad(const ScanArgs &a, hipStream_t s) {
    Dispatch go(a, s);
    if (!EXT && !ZOH && a.n_full > 0) {
        const int64_t split = a.n_cblk * a.Bsz - a.n_full;
        go(true, quad_split_kernel<IO, VEC>, dim3(static_cast<unsigned>(a.n_full + 2 * split)),
           dim3(64), a);
        return hipGetLastError();
    }
    const dim3 grid(static_cast<unsigned>(a.n_cblk * a.Bsz), static_cast<unsigned>(a.J));
    if (a.flags) {
        go(true, quad_fused_kernel<IO, VEC, EXT, ZOH>, grid, dim3(64), a);
        return hipGetLastError();
    }
    if (a.J > 1) {
        const dim3 agrid(static_cast<unsigned>(a.n_cblk * a.Bsz), static_cast<unsigned>(a.J - 1));
        go(false, quad_kernel<IO, false, VEC, EXT, ZOH>, agrid, dim3(64), a);
        if (a.hstart) {   // otherwise every chunk folds its predecessors itself
            const int64_t waves = a.Bsz * a.D * a.G;
            go(false, carry_kernel, dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256), a);
        }
    }
    go(true, quad_kernel<IO, true, VEC, EXT, ZOH>, grid, dim3(64), a);
    return hipGetLastError();
}

template <class IO, int GW, bool VEC, bool EXT, bool ZOH>
static hipError_t launch_group(const ScanArgs &a, hipStream_t s) {
    Dispatch go(a, s);
    const dim3 grid(static_cast<unsigned>(a.n_cblk * a.Bsz), static_cast<unsigned>(a.J));
    if (a.J > 1) {
        const dim3 agrid(static_cast<unsigned>(a.n_cblk * a.Bsz), static_cast<unsigned>(a.J - 1));
        go(false, group_kernel<IO, GW, false, VEC, EXT, ZOH>, agrid, dim3(64 * GW), a);
        if (a.hstart) {
            const int64_t waves = a.Bsz * a.D * a.G;
            go(false, carry_kernel, dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256), a);
        }
    }
    go(true, group_kernel<IO, GW, true, VEC, EXT, ZOH>, grid, dim3(64 * GW), a);
    return hipGetLastError();
}

template <class IO, int GW>
static hipError_t launch_group_vec(const ScanArgs &a, hipStream_t s) {
    // 4-token pieces of B and C need their rows and base pointers aligned
    auto al = [](const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
    const bool vec = a.L % 4 == 0 && al(a.B) && al(a.C);
    if (a.zoh)
        return vec ? launch_group<IO, GW, true, true, true>(a, s)
                   : launch_group<IO, GW, false, true, true>(a, s);
    if (a.cu || a.conv_w > 0)
        return vec ? launch_group<IO, GW, true, true, false>(a, s)
                   : launch_group<IO, GW, false, true, false>(a, s);
    return vec ? launch_group<IO, GW, true, false, false>(a, s)
               : launch_group<IO, GW, false, false, false>(a, s);
}

template <class IO>
static hipError_t launch_scan_io(const ScanArgs &a, hipStream_t s) {
    if (a.quad) {
        constexpr int VW = Seg<IO>::VW;
        auto al = [](const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
        const bool vec = a.L % VW == 0 && al(a.u) && al(a.delta) && al(a.y) &&
                         (!a.z || al(a.z)) && al(a.B) && al(a.C) && quad_views_fit<IO>(a);
        if (a.zoh)
            return vec ? launch_quad<IO, true, true, true>(a, s)
                       : launch_quad<IO, false, true, true>(a, s);
        if (a.cu || a.conv_w > 0)
            return vec ? launch_quad<IO, true, true, false>(a, s)
                       : launch_quad<IO, false, true, false>(a, s);
        return vec ? launch_quad<IO, true, false, false>(a, s)
                   : launch_quad<IO, false, false, false>(a, s);
    }
    switch (a.G / 2) {   // wavefronts of 32 states; the plan pads to a power of two
        case 1: return launch_group_vec<IO, 1>(a, s);
        case 2: return launch_group_vec<IO, 2>(a, s);
        case 4: return launch_group_vec<IO, 4>(a, s);
        case 8: return launch_group_vec<IO, 8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <class IO>
static hipError_t launch_agg_io(const ScanArgs &a, hipStream_t s) {
    constexpr int VW = Seg<IO>::VW;
    auto al = [](const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
    const bool vec = a.L % VW == 0 && al(a.u) && al(a.delta) && al(a.B) && al(a.C) &&
                     quad_views_fit<IO>(a);
    const dim3 agrid(static_cast<unsigned>(a.n_cblk * a.Bsz), static_cast<unsigned>(a.J - 1));
    if (a.zoh) {   // zero-order hold: the extended ZOH instance
        if (vec)
            hipLaunchKernelGGL((quad_kernel<IO, false, true, true, true>), agrid, dim3(64), 0, s, a);
        else
            hipLaunchKernelGGL((quad_kernel<IO, false, false, true, true>), agrid, dim3(64), 0, s, a);
    } else if (a.cu) {   // packed sequences: the extended instance
        if (vec)
            hipLaunchKernelGGL((quad_kernel<IO, false, true, true, false>), agrid, dim3(64), 0, s, a);
        else
            hipLaunchKernelGGL((quad_kernel<IO, false, false, true, false>), agrid, dim3(64), 0, s, a);
    } else if (vec) {
        hipLaunchKernelGGL((quad_kernel<IO, false, true, false, false>), agrid, dim3(64), 0, s, a);
    } else {
        hipLaunchKernelGGL((quad_kernel<IO, false, false, false, false>), agrid, dim3(64), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_scan_agg(const ScanArgs &a, hipStream_t s) {
    if (!a.quad || a.J < 2) return hipErrorInvalidValue;
    return a.bf16 ? launch_agg_io<BF16>(a, s) : launch_agg_io<F32>(a, s);
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
