// ssm_tscan.hip -- the in-wave time-parallel selective scan (d_state <= 16).
//
// Sources (web pages on the Mamba selective scan):
//   "From FlashAttention to Mamba" (kj168168) -- §三.2: the recurrence
//     h_t = a_t h_{t-1} + b_t is a prefix scan under the associative
//     composition (a2, b2) o (a1, b1) = (a1 a2, a2 b1 + b2), computable in
//     logarithmic depth;
//   ufo.work article "Mamba hardware-aware operator fusion and selective-scan
//     parallelisation" -- §1.1 recurrence and discretisation, §2.1 every
//     element-wise step fused into the one kernel, §3.1 the sequence cut into
//     chunks that are scanned locally, whose transfer operators are combined
//     and whose start states are then broadcast;
//   SSM engineering essay (discosf.com) -- §1.1 skip term D, §1.2 the
//     zero-order-hold input term, §1.3 softplus step size.
//
// When the channels of a call are too few for one wavefront per 16 channels
// to fill the chip, the serial mapping of quad_kernel needs sequence chunks
// on separate workgroups, and every chunk but the last is then scanned twice
// (once for its transfer operator, once for y), every exponential included.
// This kernel gets the time parallelism inside the wavefront instead, and
// evaluates each exp(dt A) once:
//
//   one wavefront = one channel; lane l holds states 4q .. 4q+3 (q = l / 16,
//   its row) of time segment s = l % 16.  The sequence is walked in tiles of
//   K = 16 TS tokens; segment s of a tile is its tokens s TS .. s TS + TS-1.
//   Per tile:
//   (a) per-token work, 64 lanes x K/64 tokens: dt = softplus(delta + bias),
//       w = dt u, D u and silu(z); dt and w go to LDS, D u and silu(z) stay
//       in the converting lane for (e).  The workgroup's 4 wavefronts (4
//       channels of one batch row) stage the tile's B and C rows in LDS
//       together, state-major, one segment row per thread;
//   (b) local scan: for its TS tokens and 4 states the lane forms
//       dA = exp2(dt A log2 e) and dBu = w B (times the zero-order-hold
//       factor), keeps both in VGPRs, and folds them from a zero state into
//       the segment's operator (a, b): b = dA b + dBu, a = exp(A sum dt);
//   (c) the inclusive scan of the 16 segment operators of each row with the
//       composition above: four wave64 DPP steps (row_shr:1, 2, 4, 8);
//   (d) the state entering each segment: the incoming tile state h_c carried
//       through the prefix (a h_c + b, shifted one segment by row_shr:1);
//       the tile's final state, broadcast from segment 15 (row_newbcast:15),
//       is the next tile's h_c -- the tiles are chunks of K tokens whose
//       transfer operators carry the state from one to the next;
//   (e) replay from the VGPRs: h = dA h + dBu and C.h per token; the four
//       rows' partial sums of 4 tokens meet in a transposing butterfly of
//       v_permlane16_swap / v_permlane32_swap; y = (C.h + D u) silu(z) is
//       written by the lane that converted the token, coalesced.
// Per (token, state) this is 7 FMA-slots of the method's arithmetic (exp
// counted as 2, the segment fold as 1 more than the serial recurrence) plus
// about 1 for the scan and carry amortised over the segment, against about
// 11 for the two-pass chunked schedule.  Each input is read once; there is
// no workspace.
#include <type_traits>

#include <hip/hip_ext.h>

#include "ssm_common.h"
#include "ssm_launch.h"
#include "ssm_seq.h"

namespace ssm {

namespace {

// DPP within rows of 16 lanes.  `old` is what a lane whose source lies
// outside its row receives (row_shr) -- the identity of the operand.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float old, float src) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, 0xF, 0xF, false));
}
constexpr int kRowShr1 = 0x111;
constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int kRowNewBcast15 = 0x15F;

// One step of the inclusive scan along a row, for the 4 states of a lane:
// with (a', b') the operator of the lane SHR places back in the row,
// (a, b) := (a', b') then (a, b), i.e. b += a b', a *= a'.  The DPP operand
// is folded into v_fmac_f32 / v_mul_f32; with bound_ctrl off a lane whose
// source lies outside the row is not written and keeps (a, b), which is the
// composition with the identity.  (The compiler keeps the identity in a
// register of its own and adds two moves per state and step.)  s_nop 1
// gives the two wait states that a DPP read needs after a VALU write of the
// same register; inside the block every DPP source was written at least
// four instructions earlier.
#define SSM_TSCAN_STEP(SHR, a, b)                                                          \
    asm volatile(                                                                          \
        "s_nop 1\n\t"                                                                       \
        "v_fmac_f32_dpp %4, %4, %0 row_shr:" #SHR " row_mask:0xf bank_mask:0xf\n\t"          \
        "v_fmac_f32_dpp %5, %5, %1 row_shr:" #SHR " row_mask:0xf bank_mask:0xf\n\t"          \
        "v_fmac_f32_dpp %6, %6, %2 row_shr:" #SHR " row_mask:0xf bank_mask:0xf\n\t"          \
        "v_fmac_f32_dpp %7, %7, %3 row_shr:" #SHR " row_mask:0xf bank_mask:0xf\n\t"          \
        "v_mul_f32_dpp %0, %0, %0 row_shr:" #SHR " row_mask:0xf bank_mask:0xf\n\t"           \
        "v_mul_f32_dpp %1, %1, %1 row_shr:" #SHR " row_mask:0xf bank_mask:0xf\n\t"           \
        "v_mul_f32_dpp %2, %2, %2 row_shr:" #SHR " row_mask:0xf bank_mask:0xf\n\t"           \
        "v_mul_f32_dpp %3, %3, %3 row_shr:" #SHR " row_mask:0xf bank_mask:0xf"                 \
        : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), \
          "+v"(b[3]))

// NE consecutive elements of a row as raw 32-bit words (two bf16 per word).
template <class IO, int NE>
struct Raw {
    static constexpr int NW = NE * static_cast<int>(sizeof(typename IO::T)) / 4;
    uint32_t w[NW];
};

// Load NE elements at token t of a row (row = the row's first element) as
// raw words, one element access each, the token index clamped to L - 1 (the
// element path: rows not in 16-byte pieces; the vector path reads through
// buffer views, below).
template <class IO, int NE>
__device__ __forceinline__ void load_raw(const typename IO::T *__restrict__ row, int t, int L,
                                         Raw<IO, NE> &r) {
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const int tc = t + i < L ? t + i : L - 1;
        if constexpr (std::is_same<IO, F32>::value) {
            r.w[i] = __float_as_uint(row[tc]);
        } else {
            const uint32_t v = row[tc];
            if (i % 2 == 0) r.w[i / 2] = v; else r.w[i / 2] |= v << 16;
        }
    }
}

// NE elements at byte offset off of a buffer view, as raw words: one vector
// access per 16 bytes, all in or all past the view's range (runs are aligned
// to their size and ranges are whole rows); past it they read as zeros.
template <class IO, int NE>
__device__ __forceinline__ void load_view(Rsrc v, uint32_t off, Raw<IO, NE> &r) {
    using R = Raw<IO, NE>;
    if constexpr (R::NW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < R::NW / 4; ++i) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(v, off + 16 * i, 0, 0);
            r.w[4 * i] = x[0]; r.w[4 * i + 1] = x[1]; r.w[4 * i + 2] = x[2]; r.w[4 * i + 3] = x[3];
        }
    } else if constexpr (R::NW == 2) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(v, off, 0, 0);
        r.w[0] = x[0]; r.w[1] = x[1];
    } else {
        r.w[0] = __builtin_amdgcn_raw_buffer_load_b32(v, off, 0, 0);
    }
}

// NE values to byte offset off of a buffer view, converted to the I/O type
// (bf16: round to nearest even); a run past the range is dropped.
template <class IO, int NE>
__device__ __forceinline__ void store_view(Rsrc v, uint32_t off, const float (&x)[NE]) {
    constexpr bool F = std::is_same<IO, F32>::value;
    constexpr int NW = F ? NE : NE / 2;
    uint32_t w[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i)
        w[i] = F ? __float_as_uint(x[i]) : Seg<BF16>::pk(x[2 * i], x[2 * i + 1]);
    if constexpr (NW == 4) {
        using V4 = __attribute__((ext_vector_type(4))) unsigned int;
        __builtin_amdgcn_raw_buffer_store_b128(V4{w[0], w[1], w[2], w[3]}, v, off, 0, 0);
    } else if constexpr (NW == 2) {
        using V2 = __attribute__((ext_vector_type(2))) unsigned int;
        __builtin_amdgcn_raw_buffer_store_b64(V2{w[0], w[1]}, v, off, 0, 0);
    } else {
        static_assert(NW == 1, "runs of 1, 2 or 4 words");
        __builtin_amdgcn_raw_buffer_store_b32(w[0], v, off, 0, 0);
    }
}

template <class IO, int NE>
__device__ __forceinline__ void unpack_raw(const Raw<IO, NE> &r, float (&o)[NE]) {
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        if constexpr (std::is_same<IO, F32>::value)
            o[i] = __uint_as_float(r.w[i]);
        else
            o[i] = (i % 2 == 0) ? __uint_as_float(r.w[i / 2] << 16)
                                : __uint_as_float(r.w[i / 2] & 0xffff0000u);
    }
}

// Store NE values at token t of a row, converting to the I/O type (bf16:
// round to nearest even), one element store each; tokens at or past L are not
// written (the element path; the vector path stores through a buffer view).
template <class IO, int NE>
__device__ __forceinline__ void store_run(typename IO::T *__restrict__ p, size_t base, int64_t t,
                                          int64_t L, const float (&v)[NE]) {
#pragma unroll
    for (int i = 0; i < NE; ++i)
        if (t + i < L) IO::store(p, base + t + i, v[i]);
}

template <int N>
__device__ __forceinline__ void lds_read(const float *p, float (&o)[N]) {
    static_assert(N % 4 == 0, "LDS runs of whole float4");
#pragma unroll
    for (int i = 0; i < N; i += 4) {
        const float4 v = *reinterpret_cast<const float4 *>(p + i);
        o[i] = v.x; o[i + 1] = v.y; o[i + 2] = v.z; o[i + 3] = v.w;
    }
}

template <int N>
__device__ __forceinline__ void lds_write(float *p, const float (&v)[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4)
            *reinterpret_cast<float4 *>(p + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
    } else if constexpr (N == 2) {
        *reinterpret_cast<float2 *>(p) = make_float2(v[0], v[1]);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) p[i] = v[i];
    }
}

}  // namespace

constexpr int kTsSegs = 16;         // time segments per tile (lanes of a row)

// Wavefronts (channels) per workgroup: the B and C rows of a tile are
// staged once for all of them.  Segments of 16 tokens: 8 wavefronts, two per
// SIMD of a CU, the B and C tiles double-buffered (one barrier per tile) and
// two tiles' inputs in flight for bfloat16 I/O; segments of 8: 4 wavefronts,
// so that three workgroups fill a CU at three wavefronts per SIMD, with
// single buffers.
#ifndef SSM_TS16_WAVES
#define SSM_TS16_WAVES 8
#endif
#ifndef SSM_TS16_BUFFERS
#define SSM_TS16_BUFFERS 2
#endif
#ifndef SSM_TS16_PREFETCH_BF16
#define SSM_TS16_PREFETCH_BF16 2
#endif
#ifndef SSM_TS16_AHEAD
#define SSM_TS16_AHEAD 1
#endif
template <int TS>
constexpr int ts_waves() { return TS == 16 ? SSM_TS16_WAVES : 4; }

// AHEAD (segments of 16, two tiles in flight): each tile stages the next
// tile's B and C rows into the third of three LDS buffers, and the wavefronts order their accesses
// through progress counters in LDS instead of a barrier per tile (see the
// tile loop).
template <class IO, int TS>
struct TsShape {
    static constexpr int W = ts_waves<TS>();
    static constexpr int PF = (TS == 16 && std::is_same<IO, BF16>::value) ? SSM_TS16_PREFETCH_BF16
                                                                          : 1;   // tiles in flight
    // (staging one tile ahead takes the next tile's register set: two in flight)
    static constexpr bool AHEAD = TS == 16 && PF == 2 && SSM_TS16_AHEAD;
    static constexpr int NBUF = AHEAD ? 3 : TS == 16 ? SSM_TS16_BUFFERS : 1;   // B/C tile buffers
};

// TS: tokens per segment (8 or 16); tiles of 16 TS tokens.
// Occupancy: TS = 16 keeps 128 VGPRs of dA/dBu (two wavefronts per SIMD),
// TS = 8 keeps 64 (three per SIMD).
// GT: with the silu gate (z given); SPL: softplus on the step size; CK: the
// replay also writes the state entering every kBwdTile-token tile
// (a.ckpt, for the backward pass).  All are template flags so that the tile
// loop holds no branch on them.
template <class IO, int TS, bool VEC, bool ZOH, bool GT, bool SPL, bool CK>
__global__ __launch_bounds__(64 * ts_waves<TS>(), TS == 8 ? 3 : 2) void tscan_kernel(ScanArgs a) {
    using IT = typename IO::T;
    using SH = TsShape<IO, TS>;
    constexpr int W = SH::W;
    constexpr int NBUF = SH::NBUF;
    constexpr int PF = SH::PF;
    constexpr bool AHEAD = SH::AHEAD;
    constexpr int S = kTsSegs;
    constexpr int K = S * TS;           // tokens per tile
    constexpr int SP = TS + 4;          // LDS segment row, padded (bank spread)
    constexpr int RS = S * SP;          // LDS row of one state (or channel): the tile
    constexpr int PT = K / kWave;       // tokens per lane in the per-token stages
    constexpr int TPR = 4 * W;          // staging threads per state row
    constexpr int BT = K / TPR;         // tokens of B (and C) per staging thread
    static_assert(TS % 4 == 0 && PT % 2 == 0 && PT * 4 == TS, "tile shape");
    static_assert(BT % 4 == 0 && TS % BT == 0, "staging pieces within a segment");
    static_assert(TS % kBwdTile == 0, "checkpoint tiles start on segment tokens");

    __shared__ __attribute__((aligned(16))) float sB[NBUF * 16 * RS];
    __shared__ __attribute__((aligned(16))) float sC[NBUF * 16 * RS];
    __shared__ __attribute__((aligned(16))) float sDT[W * RS];
    __shared__ __attribute__((aligned(16))) float sW[W * RS];
    __shared__ __attribute__((aligned(16))) float sY[W * RS];
    // AHEAD: per wavefront, its count of ordering events (see the tile loop)
    __shared__ int sEv[W];

    const IT *__restrict__ u = static_cast<const IT *>(a.u);
    const IT *__restrict__ dl = static_cast<const IT *>(a.delta);
    const IT *__restrict__ z = static_cast<const IT *>(a.z);
    const IT *__restrict__ Bm = static_cast<const IT *>(a.B);
    const IT *__restrict__ Cm = static_cast<const IT *>(a.C);
    IT *__restrict__ y = static_cast<IT *>(a.y);

    const int tid = threadIdx.x;
    // wavefront: channel of the block (uniform, so that the row views
    // below live in scalar registers)
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int q = lane >> 4;                    // row: states 4q .. 4q+3
    const int s = lane & 15;                    // time segment
    const int64_t b = blockIdx.x / a.n_cblk;
    const int64_t d = static_cast<int64_t>(blockIdx.x % a.n_cblk) * W + wv;
    const bool ch_ok = d < a.D;                 // wave-uniform
    const int64_t dc = ch_ok ? d : a.D - 1;
    const int64_t L = a.L;
    const size_t rbase = (static_cast<size_t>(b) * a.D + dc) * L;

    // per-token stage: lane covers tokens lane PT .. lane PT + PT-1 of the
    // tile, in segment lane / 4
    const int pseg = lane >> 2;
    const int poff = pseg * SP + (lane & 3) * PT;
    // B/C staging: thread covers tokens bt0 .. bt0 + BT-1 of state row bn,
    // inside one segment
    const int bn = tid / TPR;
    const int bt0 = (tid % TPR) * BT;
    const int boff = bn * RS + (bt0 / TS) * SP + bt0 % TS;
    const bool bn_ok = bn < a.N;
    const size_t sbase = (static_cast<size_t>(b) * a.N + (bn_ok ? bn : a.N - 1)) * L;
    const float rbias = a.delta_bias ? a.delta_bias[dc] : 0.0f;
    const float rD = a.Dskip ? a.Dskip[dc] : 0.0f;
    float A2[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int n = 4 * q + k;
        const float v = a.A[dc * a.N + (n < a.N ? n : a.N - 1)];
        A2[k] = n < a.N ? v * kLog2e : 0.0f;
    }
    // the state entering the tile (the start state at token 0)
    float hc[4];
    load_start_state<4>(a, b, dc, ch_ok, 4 * q, hc);

    float *sdt = sDT + wv * RS;
    float *sw = sW + wv * RS;
    float *sy = sY + wv * RS;
    // CK: this lane's states 4q .. 4q+3 in the channel's checkpoint row
    // (batch, d_inner, n_ck, 16); states past N hold zero, as h does there
    float *const ckrow =
        (CK && ch_ok) ? a.ckpt + (static_cast<size_t>(b) * a.D + d) * a.n_ck * 16 + 4 * q : nullptr;

    // a tile's inputs in registers (raw words), loaded PF tiles ahead
    struct Regs {
        Raw<IO, PT> u, d, z;
        Raw<IO, BT> b, c;
    };
    // row pointers of this lane's pieces (token indices fit in int: L <= 2^25)
    const IT *u_row = u + rbase;
    const IT *d_row = dl + rbase;
    // without a gate z reads u's row again (cached, unused): the same loads on
    // every path keep the compiler's count of loads in flight exact
    const IT *z_row = GT ? z + rbase : u_row;
    const IT *b_row = Bm + sbase;
    const IT *c_row = Cm + sbase;
    const int Li = static_cast<int>(L);
    // VEC: the tile loads and the y stores go through wave-uniform buffer
    // views: the channel's rows of u, delta, z and y (L elements each) and
    // the batch row's N rows of B and C, past which rows n >= N read as
    // zeros.  A lane's byte offsets are fixed plus the tile's first token;
    // tokens at or past L read as zeros and their y stores are dropped.
    // (The launch takes this path only when the offsets, below 16 L + 3 K
    // elements, stay under 2^31 bytes.)
    constexpr uint32_t ESZ = sizeof(IT);
    const uint64_t row_bytes = VEC ? static_cast<uint64_t>(L) * ESZ : 0;
    const Rsrc v_u = view(u_row, row_bytes), v_d = view(d_row, row_bytes);
    const Rsrc v_z = view(z_row, row_bytes), v_y = view(y + rbase, row_bytes);
    const uint64_t bc_bytes = VEC ? static_cast<uint64_t>(a.N) * L * ESZ : 0;
    const Rsrc v_b = view(Bm + static_cast<size_t>(b) * a.N * L, bc_bytes);
    const Rsrc v_c = view(Cm + static_cast<size_t>(b) * a.N * L, bc_bytes);
    const uint32_t o_tok = static_cast<uint32_t>(lane * PT) * ESZ;
    const uint32_t o_bc = (static_cast<uint32_t>(bn) * static_cast<uint32_t>(Li) + bt0) * ESZ;
    auto load_tile = [&](Regs &r, int64_t t0) {
        const int tl = static_cast<int>(t0) + lane * PT;
        const int tb = static_cast<int>(t0) + bt0;
        const uint32_t ot = static_cast<uint32_t>(t0) * ESZ;
        // AHEAD stages B and C a tile before the tile's own loads are needed:
        // issued first, they can be waited for while u, delta and z are
        // still in flight (loads complete in issue order).  z next: the
        // compiler copies its registers at the loop's back edge, which then
        // waits for it alone.  The scheduling barriers keep that order.
        auto ld_bc = [&] {
            if constexpr (VEC) {
                load_view<IO, BT>(v_b, o_bc + ot, r.b);
                load_view<IO, BT>(v_c, o_bc + ot, r.c);
            } else {
                load_raw<IO, BT>(b_row, tb, Li, r.b);   // rows n >= N read row N-1, unused
                load_raw<IO, BT>(c_row, tb, Li, r.c);
            }
        };
        auto ld_tok = [&](Rsrc v, const IT *row, Raw<IO, PT> &x) {
            if constexpr (VEC) load_view<IO, PT>(v, o_tok + ot, x);
            else load_raw<IO, PT>(row, tl, Li, x);
        };
        if constexpr (AHEAD) {
            ld_bc();
            __builtin_amdgcn_sched_barrier(0);
            ld_tok(v_z, z_row, r.z);
            __builtin_amdgcn_sched_barrier(0);
        }
        ld_tok(v_u, u_row, r.u);
        ld_tok(v_d, d_row, r.d);
        if constexpr (!AHEAD) ld_tok(v_z, z_row, r.z);
        if constexpr (!AHEAD) ld_bc();
    };

    // This thread's pieces of a tile's B and C rows into LDS buffer nb
    // (branch-free: a branch here would make the compiler wait for every load
    // in flight); rows n >= N store B = 0 (VEC: read as zeros).
    auto stage_bc = [&](const Regs &r, const int nb) {
        float xb[BT], xc[BT];
        unpack_raw<IO, BT>(r.b, xb);
        if constexpr (!VEC) {
#pragma unroll
            for (int i = 0; i < BT; ++i) xb[i] = bn_ok ? xb[i] : 0.0f;
        }
        lds_write<BT>(sB + nb * 16 * RS + boff, xb);
        unpack_raw<IO, BT>(r.c, xc);
        lds_write<BT>(sC + nb * 16 * RS + boff, xc);
    };
    // AHEAD: wait until every wavefront's event count has reached target;
    // returns the smallest count seen.  The poll is one asm block: its loop
    // is invisible to the compiler, which would otherwise keep more of the
    // tile's values live across it (and spill them), and its LDS reads are
    // waited for inside the block.  All lanes read the same words, so the
    // test is uniform; the wavefront sleeps between polls.  The wait always
    // ends (see the tile loop); the bound on the polls is a guard only.
    static_assert(!AHEAD || W == 8, "the poll reads 8 counters");
    using LdsInt = __attribute__((address_space(3))) int;
    LdsInt *const ev_lds = (LdsInt *)sEv;
    auto wait_all = [&](const int target) -> int {
        int c0, c1, c2, c3, c4, c5, c6, c7, sm, it;
        asm volatile(
            "s_mov_b32 %[it], 0\n"
            "1:\n\t"
            "ds_read_b32 %[c0], %[ea]\n\t"
            "ds_read_b32 %[c1], %[ea] offset:4\n\t"
            "ds_read_b32 %[c2], %[ea] offset:8\n\t"
            "ds_read_b32 %[c3], %[ea] offset:12\n\t"
            "ds_read_b32 %[c4], %[ea] offset:16\n\t"
            "ds_read_b32 %[c5], %[ea] offset:20\n\t"
            "ds_read_b32 %[c6], %[ea] offset:24\n\t"
            "ds_read_b32 %[c7], %[ea] offset:28\n\t"
            "s_waitcnt lgkmcnt(0)\n\t"
            "v_min3_i32 %[c0], %[c0], %[c1], %[c2]\n\t"
            "v_min3_i32 %[c0], %[c0], %[c3], %[c4]\n\t"
            "v_min3_i32 %[c0], %[c0], %[c5], %[c6]\n\t"
            "v_min_i32 %[c0], %[c0], %[c7]\n\t"
            "s_nop 4\n\t"
            "v_readfirstlane_b32 %[sm], %[c0]\n\t"
            "s_nop 4\n\t"
            "s_cmp_ge_i32 %[sm], %[tg]\n\t"
            "s_cbranch_scc1 2f\n\t"
            "s_add_u32 %[it], %[it], 1\n\t"
            "s_cmp_lt_u32 %[it], %[lim]\n\t"
            "s_cbranch_scc0 2f\n\t"
            "s_sleep 1\n\t"
            "s_branch 1b\n"
            "2:"
            : [c0] "=&v"(c0), [c1] "=&v"(c1), [c2] "=&v"(c2), [c3] "=&v"(c3), [c4] "=&v"(c4),
              [c5] "=&v"(c5), [c6] "=&v"(c6), [c7] "=&v"(c7), [sm] "=&s"(sm), [it] "=&s"(it)
            : [ea] "v"(ev_lds), [tg] "s"(target), [lim] "s"(1 << 24)
            : "memory", "scc");
        return sm;
    };
    // AHEAD: publish this wavefront's event count once its LDS accesses
    // before it are complete (lgkmcnt(0)); every lane stores the same value.
    auto signal = [&](const int value) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0xC07F);
        reinterpret_cast<volatile LdsInt *>(ev_lds)[wv] = value;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };

    // One tile: tokens t0 .. t0 + K-1 (tile index ti), inputs in r (which
    // then takes the inputs of the tile PF tiles later).  Without AHEAD its B
    // and C rows go from r to LDS buffer nb here; with AHEAD they were staged
    // by the tile before, into buffer ti % 3, and this tile stages the next
    // one's from rn into buffer (ti + 1) % 3.
    auto tile = [&](const int64_t t0, Regs &r, Regs &rn, const int nb, auto mask_tag) {
        // MASK: a tile that reaches past L (only the last group of tiles)
        constexpr bool MASK = decltype(mask_tag)::value;
        const int ti = static_cast<int>(t0 / K);
        const int nr = AHEAD ? ti % 3 : nb;
        // barrier-ordered instances: the workgroups that share a CU (three at
        // segments of 8) get issue slots oldest first; priority falling with
        // the tiles done lets the ones behind catch up, so that they end
        // together rather than the youngest alone
        if constexpr (!AHEAD) fair_prio(ti, (L + K - 1) / K);
        float *bB = sB + nr * 16 * RS;
        float *bC = sC + nr * 16 * RS;
        // ---- (a) per-token values of this lane's tokens; B and C rows
        float du[PT], g[PT];
        {
            float xu[PT], xd[PT], xz[PT], xdt[PT], xw[PT];
            unpack_raw<IO, PT>(r.u, xu);
            unpack_raw<IO, PT>(r.d, xd);
            if (GT) unpack_raw<IO, PT>(r.z, xz);
#pragma unroll
            for (int i = 0; i < PT; ++i) {
                const float x = xd[i] + rbias;
                float dt = SPL ? softplus_f32(x) : x;
                float uu = xu[i];
                if (MASK && t0 + lane * PT + i >= L) {   // padding: identity steps
                    dt = 0.0f;
                    uu = 0.0f;
                }
                xdt[i] = dt;
                xw[i] = dt * uu;
                du[i] = rD * uu;
                g[i] = GT ? silu_f32(xz[i]) : 1.0f;
            }
            lds_write<PT>(sdt + poff, xdt);
            lds_write<PT>(sw + poff, xw);
            // the segment's sum of dt, for its decay in (c): the 4 lanes of
            // a segment add their pieces (every lane gets the same sum) and
            // store it in the padding after the segment's tokens
            float ps = xdt[0];
#pragma unroll
            for (int i = 1; i < PT; ++i) ps += xdt[i];
            ps += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ps), kQuadSwap1, 0xF, 0xF, true));
            ps += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ps), kQuadSwap2, 0xF, 0xF, true));
            sdt[pseg * SP + TS] = ps;
        }
        if constexpr (AHEAD) {
            // every wavefront has staged its pieces of this tile and is done
            // reading buffer (ti + 1) % 3, which last held tile ti - 2, before
            // it is overwritten (event count >= 2 ti; >= 1 for tile 0)
            const int slowest = wait_all(ti == 0 ? 1 : 2 * ti);
            // This wavefront's count is 2 ti + 1 (1 at tile 0).  One ahead of
            // the slowest gives way: the SIMD's instruction arbiter favours the
            // older of its wavefronts, which would otherwise run ahead until
            // it must wait, leaving its SIMD to the younger one alone.
            if (slowest < 2 * ti + 1) __builtin_amdgcn_s_setprio(0);
            else __builtin_amdgcn_s_setprio(2);
            stage_bc(rn, (ti + 1) % 3);
            signal(2 * ti + 2);
        } else {
            stage_bc(r, nb);
        }
        // the inputs of the tile PF tiles later, in flight during this one's
        // scan (addresses are clamped into the row: the same loads on every path)
        load_tile(r, t0 + PF * K);
        if constexpr (!AHEAD) {
            // with one buffer, every wavefront must be done with the previous
            // tile's B and C rows before they are overwritten: a barrier before
            // the writes above (at the end of the previous tile); with two, the
            // barrier below also orders the writes of the next tile into the
            // other buffer after every read of it during the previous tile
            __syncthreads();
        }

        // ---- (b) local scan of the segment from a zero state; dA and dBu stay
        // in VGPRs for the replay
        float eA[TS][4], eB[TS][4];
        float bs[4];
        const float dtsum = sdt[s * SP + TS];
#pragma unroll
        for (int g4 = 0; g4 < TS; g4 += 4) {
            float dt4[4], w4[4], B4[4][4];
            lds_read<4>(sdt + s * SP + g4, dt4);
            lds_read<4>(sw + s * SP + g4, w4);
#pragma unroll
            for (int k = 0; k < 4; ++k) lds_read<4>(bB + (4 * q + k) * RS + s * SP + g4, B4[k]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = g4 + j;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float xa = dt4[j] * A2[k];
                    const float e = exp2_hw(xa);
                    float v = w4[j] * B4[k][j];
                    if (ZOH) v *= zoh_phi(xa * kLn2, e);
                    eA[t][k] = e;
                    eB[t][k] = v;
                    bs[k] = t == 0 ? v : __builtin_fmaf(e, bs[k], v);
                }
            }
        }

        // ---- (c) inclusive scan of the segment operators along the row
        float as[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) as[k] = exp2_hw(A2[k] * dtsum);
        SSM_TSCAN_STEP(1, as, bs);
        SSM_TSCAN_STEP(2, as, bs);
        SSM_TSCAN_STEP(4, as, bs);
        SSM_TSCAN_STEP(8, as, bs);

        // ---- (d) state entering this segment; the next tile's state
        float h[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float hout = __builtin_fmaf(as[k], hc[k], bs[k]);
            h[k] = dpp_row<kRowShr1>(hc[k], hout);
            hc[k] = __int_as_float(
                __builtin_amdgcn_mov_dpp(__float_as_int(hout), kRowNewBcast15, 0xF, 0xF, true));
        }

        // ---- (e) replay, C.h, butterfly over the rows; y sums to LDS
#pragma unroll
        for (int g4 = 0; g4 < TS; g4 += 4) {
            float C4[4][4];
#pragma unroll
            for (int k = 0; k < 4; ++k) lds_read<4>(bC + (4 * q + k) * RS + s * SP + g4, C4[k]);
            float acc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = g4 + j;
                if constexpr (CK) {
                    if (t % kBwdTile == 0) {   // h enters token t0 + s TS + t
                        const int64_t tok = t0 + s * TS + t;
                        if (ch_ok && (!MASK || tok < L)) {
                            // segments of 8 (many channels): non-temporal
                            // stores (Mamba-130M-shaped layer with
                            // checkpoints 50 -> 40 us); segments of 16
                            // (long sequences): plain stores, faster there
                            // (705 against 720 us)
                            using F4 = __attribute__((ext_vector_type(4))) float;
                            F4 *dst = reinterpret_cast<F4 *>(ckrow + (tok / kBwdTile) * 16);
                            const F4 hv{h[0], h[1], h[2], h[3]};
                            if constexpr (TS == 8) __builtin_nontemporal_store(hv, dst);
                            else *dst = hv;
                        }
                    }
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) h[k] = __builtin_fmaf(eA[t][k], h[k], eB[t][k]);
                acc[j] = __builtin_fmaf(C4[0][j], h[0], __builtin_fmaf(C4[1][j], h[1],
                         __builtin_fmaf(C4[2][j], h[2], C4[3][j] * h[3])));
            }
            // rows (0,1) and (2,3): even rows keep tokens 0/2, odd rows 1/3;
            // then halves: rows 0,1 keep tokens 0,1, rows 2,3 tokens 2,3
            const auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[0]),
                                                              __float_as_uint(acc[1]), false, false);
            const auto s23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[2]),
                                                              __float_as_uint(acc[3]), false, false);
            const float p01 = __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
            const float p23 = __uint_as_float(s23[0]) + __uint_as_float(s23[1]);
            const auto sw32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p01),
                                                               __float_as_uint(p23), false, false);
            sy[s * SP + g4 + q] = __uint_as_float(sw32[0]) + __uint_as_float(sw32[1]);
        }

        // ---- y of this lane's tokens, coalesced
        {
            float ys[PT];
#pragma unroll
            for (int i = 0; i < PT; i += 2) {
                const float2 v = *reinterpret_cast<const float2 *>(sy + poff + i);
                ys[i] = v.x;
                ys[i + 1] = v.y;
            }
#pragma unroll
            for (int i = 0; i < PT; ++i) ys[i] = (ys[i] + du[i]) * g[i];
            if (ch_ok) {
                if constexpr (VEC) store_view<IO, PT>(v_y, o_tok + static_cast<uint32_t>(t0) * ESZ, ys);
                else store_run<IO, PT>(y, rbase, t0 + lane * PT, L, ys);
            }
        }
        if constexpr (AHEAD) signal(2 * ti + 3);   // done reading buffer ti % 3
        if (NBUF == 1) __syncthreads();   // every wavefront is done with this tile's B and C
    };

    // PF register sets, used in turn: PF tiles per iteration, so that every
    // set is named statically; the LDS buffers alternate with the tile.  The
    // loop runs whole groups of PF tiles only: its body is straight-line (no
    // padding masks, no exit in the middle), so the compiler's count of loads
    // in flight stays exact and each tile waits only for its own inputs.  The
    // last, partial group follows with masks.
    //
    // AHEAD ordering.  Each wavefront counts its events in sEv: 1 once tile
    // 0's B and C are staged, then per tile i: 2i + 2 once tile i + 1's are
    // staged, 2i + 3 once it is done reading tile i's.  Tile i > 0 waits until
    // every count is >= 2i, i.e. every wavefront has staged tile i (a count of
    // 2i or more) and is done with tile i - 2 (more than 2i - 1); tile 0 until
    // every count is >= 1 (tile 0 staged).  Then it stages
    // tile i + 1 into buffer (i + 1) % 3 (which held tile i - 2), reads tile
    // i's rows from buffer i % 3 and finishes.  A wavefront therefore runs at
    // most one tile ahead of the slowest, and the slowest, at tile j, never
    // waits: every wavefront, itself included, is at a tile j' >= j, so it
    // has finished tile j' - 1 and its count is at least 2j' + 1 (at least 1
    // at tile 0, after the prologue).  So every wait ends.
    Regs rs[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p) load_tile(rs[p], p * K);
    if constexpr (AHEAD) {
        // counters start at zero (the LDS may hold a previous workgroup's),
        // then tile 0's rows are staged
        sEv[wv] = 0;
        __syncthreads();
        stage_bc(rs[0], 0);
        signal(1);
    }
    auto nbuf = [&](int64_t tt) { return NBUF == 2 ? static_cast<int>((tt / K) & 1) : 0; };
    int64_t t0 = 0;
    for (; t0 + PF * K <= L; t0 += PF * K) {
#pragma unroll
        for (int p = 0; p < PF; ++p)
            tile(t0 + p * K, rs[p], rs[(p + 1) % PF], nbuf(t0 + p * K), std::false_type{});
    }
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        const int64_t tt = t0 + p * K;
        if (tt < L) tile(tt, rs[p], rs[(p + 1) % PF], nbuf(tt), std::true_type{});
    }

    // the state after the last token
    if (a.last_state && ch_ok && s == 0) {
        float *ls = a.last_state + (static_cast<size_t>(b) * a.D + d) * a.N;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (4 * q + k < a.N) ls[4 * q + k] = hc[k];
    }
}

template <class IO, int TS, bool VEC, bool ZOH, bool GT, bool SPL, bool CK>
static hipError_t launch_tscan_ck(const ScanArgs &a, hipStream_t s) {
    constexpr int W = TsShape<IO, TS>::W;
    const dim3 grid(static_cast<unsigned>(a.n_cblk * a.Bsz));
    const dim3 block(64 * W);
    if (a.ev_begin && a.ev_end)
        hipExtLaunchKernelGGL((tscan_kernel<IO, TS, VEC, ZOH, GT, SPL, CK>), grid, block, 0, s,
                              a.ev_begin, a.ev_end, 0, a);
    else
        hipLaunchKernelGGL((tscan_kernel<IO, TS, VEC, ZOH, GT, SPL, CK>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <class IO, int TS, bool VEC, bool ZOH, bool GT, bool SPL>
static hipError_t launch_tscan_one(const ScanArgs &a, hipStream_t s) {
    return a.ckpt ? launch_tscan_ck<IO, TS, VEC, ZOH, GT, SPL, true>(a, s)
                  : launch_tscan_ck<IO, TS, VEC, ZOH, GT, SPL, false>(a, s);
}

template <class IO, int TS, bool VEC>
static hipError_t launch_tscan_zoh(const ScanArgs &a0, hipStream_t s) {
    constexpr int W = TsShape<IO, TS>::W;
    ScanArgs a = a0;
    a.n_cblk = (a.D + W - 1) / W;      // workgroups of W channels per batch row
    if (a.n_cblk * a.Bsz > static_cast<int64_t>(UINT32_MAX)) return hipErrorInvalidConfiguration;
    const bool gt = a.z != nullptr, sp = a.softplus != 0;
    if (a.zoh) {
        if (gt) return sp ? launch_tscan_one<IO, TS, VEC, true, true, true>(a, s)
                          : launch_tscan_one<IO, TS, VEC, true, true, false>(a, s);
        return sp ? launch_tscan_one<IO, TS, VEC, true, false, true>(a, s)
                  : launch_tscan_one<IO, TS, VEC, true, false, false>(a, s);
    }
    if (gt) return sp ? launch_tscan_one<IO, TS, VEC, false, true, true>(a, s)
                      : launch_tscan_one<IO, TS, VEC, false, true, false>(a, s);
    return sp ? launch_tscan_one<IO, TS, VEC, false, false, true>(a, s)
              : launch_tscan_one<IO, TS, VEC, false, false, false>(a, s);
}

template <class IO>
static hipError_t launch_tscan_io(const ScanArgs &a, hipStream_t s) {
    auto al = [](const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
    // The vector path reads B and C through one view per batch row, at byte
    // offsets below (16 L + 3 K) elements (state rows up to 15, tiles loaded
    // up to two ahead of the last): they must stay below 2^31.
    const bool vec = a.L % 16 == 0 && al(a.u) && al(a.delta) && al(a.y) && (!a.z || al(a.z)) &&
                     al(a.B) && al(a.C) &&
                     (16 * static_cast<uint64_t>(a.L) + 1024) * sizeof(typename IO::T) < (1ull << 31);
    if (a.tile_ts == 16)
        return vec ? launch_tscan_zoh<IO, 16, true>(a, s) : launch_tscan_zoh<IO, 16, false>(a, s);
    if (a.tile_ts == 8)
        return vec ? launch_tscan_zoh<IO, 8, true>(a, s) : launch_tscan_zoh<IO, 8, false>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_tscan(const ScanArgs &a, hipStream_t s) {
    return a.bf16 ? launch_tscan_io<BF16>(a, s) : launch_tscan_io<F32>(a, s);
}

}  // namespace ssm
