// ssm_api.hip -- the C ABI of libssm: validation, planning, workspace layout
// and launch.  Declarations and the contract of every entry point are in
// include/ssm.h.
#include "ssm.h"

#include <hip/hip_runtime.h>
#include <limits.h>

#include <atomic>
#include <chrono>
#include <mutex>

#include "ssm_launch.h"

namespace {

using ssm::ScanArgs;

constexpr int64_t kMaxGridY = 65535;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Dense-shape sanity: every product we index with must fit in int64 and the
// grid sizes in 32 bits.
bool dims_ok(int64_t a, int64_t b, int64_t c) {
    if (a < 0 || b < 0 || c < 0) return false;
    const double p = static_cast<double>(a) * static_cast<double>(b) * static_cast<double>(c);
    return p < 9.0e18;
}

struct Plan {
    int G = 1;            // groups of 16 states in a padded state row
    int64_t K = 0;        // chunk length
    int64_t J = 1;        // chunks
    int64_t n_cblk = 0;   // blocks of 16 channels per batch row
    int quad = 0;         // d_state <= 16: quad-row kernel
    int fold = 0;         // chunks fold their predecessors' operators (no carry kernel)
    int fused = 0;        // one launch: chunks publish operators and wait for each other
    int tile_ts = 0;      // > 0: in-wave scan (tscan_kernel), chunks of 16 tile_ts tokens in
                          // sequence on one wavefront per channel, segments of tile_ts tokens
    int64_t split_full = 0;   // > 0: quad_split_kernel, blocks past this many in two chunks
    size_t off_hend = 0, off_dtsum = 0, off_keep = 0, off_hstart = 0, off_flags = 0, bytes = 0;
};

constexpr uint32_t kKnownFlags = SSM_FLAG_ZOH | SSM_FLAG_INDEPENDENT_CHUNKS;

ssm_status check_desc(const ssm_desc *d) {
    if (!d) return SSM_ERR_NULL_ARG;
    if (d->batch < 0 || d->d_inner < 0 || d->seqlen < 0) return SSM_ERR_BAD_SHAPE;
    if (d->d_state < 1 || d->d_state > SSM_MAX_D_STATE) return SSM_ERR_UNSUPPORTED;
    if (d->io_dtype != SSM_F32 && d->io_dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
    if ((d->flags & ~kKnownFlags) != 0 || d->reserved != 0) return SSM_ERR_UNSUPPORTED;
    if (d->seqlen > SSM_MAX_SEQLEN) return SSM_ERR_UNSUPPORTED;
    if (!dims_ok(d->batch, d->d_inner, d->seqlen > 0 ? d->seqlen : 1)) return SSM_ERR_BAD_SHAPE;
    if (!dims_ok(d->batch, d->d_inner, d->d_state)) return SSM_ERR_BAD_SHAPE;
    return SSM_OK;
}

// Waves wanted in flight: two per SIMD on 256 CUs x 4 SIMDs.
constexpr int64_t kTargetWaves = 2048;
constexpr int64_t kEnoughWaves = 1024;
// The quad path runs its chunks in one launch (each chunk publishes its
// operator and waits for its predecessors') from this chunk length on.
// Measured on MI355X: at 4096-token chunks (1 x 2048 channels x 64 Ki tokens,
// bf16) one launch takes 934 us against 974-1029 us for the two passes; at
// 128-192 token chunks (2 x 1536 channels x 2048 tokens, fp32) it is slower
// (74-76 us against 66-70 us for the two passes with fair priorities): with
// short chunks the waits of the younger chunks cost more than the saved
// kernel boundary gains.
constexpr int64_t kFusedMinChunk = 1024;
constexpr int64_t kMinAutoChunk = 64;
// Up to this many chunks, each chunk of the quad path folds the transfer
// operators of the chunks before it (at most this many exp per state) instead
// of waiting for a separate carry kernel.
constexpr int64_t kFoldMaxChunks = 32;
// Longest wait of a chunk for its predecessors' operators: 20 ms of the
// 100 MHz real-time clock.
constexpr uint64_t kMaxSpinTicks = 2000000;
// SIMDs of the chip: 256 CUs x 4.
constexpr int64_t kSimds = 1024;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Chunk length of the two-pass schedule of the d_state <= 16 path, for
// `waves` wavefronts per chunk: among J0 .. 2 J0 chunks (J0 puts kTargetWaves
// in flight), the count whose busiest SIMD scans the fewest tokens, both
// passes counted.  A pass's wavefronts spread evenly over the SIMDs and share
// each one fairly (quad_kernel lowers its priority as it advances), so the
// pass takes about ceil(wavefronts / kSimds) chunk lengths; the aggregate
// pass, over chunks 0 .. J-2, costs about 4/5 of the y pass per token.
// Measured on MI355X (2 x 1536 channels x 2048 tokens, fp32, both passes):
// 128-token chunks, three wavefronts on every SIMD, 66 us; 96, 160 and 192
// tokens 71-75 us.
int64_t quad_auto_chunk(int64_t L, int64_t waves) {
    const int64_t J0 = ceil_div(kTargetWaves, waves);
    int64_t best_k = L, best_cost = -1;
    for (int64_t J = J0; J <= 2 * J0; ++J) {
        int64_t k = ceil_div(ceil_div(L, J), 16) * 16;
        if (k < kMinAutoChunk) k = kMinAutoChunk;
        if (k > L) k = L;
        const int64_t nj = ceil_div(L, k);
        const int64_t cost = k * (5 * ceil_div(waves * nj, kSimds) +
                                  4 * ceil_div(waves * (nj - 1), kSimds));
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best_k = k;
        }
    }
    return best_k;
}

// The in-wave scan (tscan_kernel): one wavefront per channel, the time
// parallelism inside it.  Chosen by the library when one wavefront per 16
// channels would leave the chip short of wavefronts (so that the serial
// mapping would need chunks on separate workgroups, scanned twice) while one
// wavefront per channel gives at least one per SIMD; up to kTsMaxRows
// channels (about 2.7 rounds of three wavefronts per SIMD), above which two
// passes over few chunks cost less than the in-wave scan's extra work.
// Segments of 16 tokens (chunks of 256) hold two wavefronts per SIMD,
// segments of 8 (chunks of 128) three.
constexpr int64_t kTsMinRows = 1024;
constexpr int64_t kTsMaxRows = 8192;
constexpr int64_t kTsRows16 = 2048;
// Fewer channels and a short sequence (up to kTsShortL tokens): one launch of
// the in-wave scan at segments of 8 also beats the two passes that the serial
// mapping needs to fill the chip (measured for 64 to 1000 channels: 8-15 us
// against 17-24 us up to 1024 tokens; about even at 2048, behind at 4096).
constexpr int64_t kTsShortL = 1024;

// fwd: the plan of a forward scan, which may run the chunked quad path as
// one launch (long chunks) and, for calls without packed sequences or the
// fused convolution (lean), the in-wave scan or the balanced serial walks
// (both write checkpoints when asked).  The backward, which reuses the
// chunk-aggregate pass on its own, passes false.
ssm_status make_plan(const ssm_desc *d, Plan *p, bool fwd = true, bool lean = true) {
    const ssm_status st = check_desc(d);
    if (st != SSM_OK) return st;
    if (d->chunk_size < 0 || (d->chunk_size > 0 && d->chunk_size % 16 != 0))
        return SSM_ERR_BAD_SHAPE;
    const int64_t L = d->seqlen;
    p->quad = d->d_state <= 16;
    int GW = 1;   // wavefronts of 32 states (group_kernel), a power of two
    while (32 * GW < d->d_state) GW <<= 1;
    const int G = p->quad ? 1 : 2 * GW;
    p->G = G;
    p->n_cblk = (d->d_inner + 15) / 16;
    if (L == 0 || d->batch * d->d_inner == 0) {
        p->K = L; p->J = L > 0 ? 1 : 0; p->bytes = 0;
        return SSM_OK;
    }
    const int64_t rows = d->batch * d->d_inner;
    const bool ts_ok = fwd && lean && p->quad;
    if (ts_ok && (d->chunk_size == 128 || d->chunk_size == 256)) {
        // chunks of 128 or 256 tokens run in sequence on a wavefront per channel
        p->tile_ts = d->chunk_size / 16;
    } else if (ts_ok && d->chunk_size == 0 && d->batch * p->n_cblk < kEnoughWaves &&
               rows >= kTsMinRows && rows <= kTsMaxRows && L > 64) {
        p->tile_ts = rows <= kTsRows16 ? 16 : 8;
    } else if (ts_ok && d->chunk_size == 0 && rows < kTsMinRows && L > 64 && L <= kTsShortL) {
        p->tile_ts = 8;
    }
    if (p->tile_ts > 0) {
        p->K = 16 * p->tile_ts < L ? 16 * p->tile_ts : L;
        p->J = 1;
        p->bytes = 0;
        return SSM_OK;
    }
    // One wavefront per 16-channel block, whole sequence, leaves the SIMDs
    // unevenly loaded when the blocks are not a whole number of rounds: then
    // the blocks past the last whole round run as two chunks each, on two
    // wavefronts that fill the next slot of every SIMD (quad_split_kernel).
    // The first chunk scans its tokens twice (aggregate, then y; about 1.8 y
    // passes), so it takes 1/2.8 of the sequence and both chunks cost about
    // the same: a SIMD then scans about 0.64 of a block instead of a whole
    // one on top of its whole rounds.  Used when that shortens the busiest
    // SIMD's work by at least a tenth, three wavefronts per SIMD hold the
    // grid, and rows take whole 16-byte pieces (the element path needs more
    // registers than three wavefronts per SIMD leave it).
    const int64_t vw = d->io_dtype == SSM_BF16 ? 8 : 4;
    if (fwd && lean && p->quad && (d->flags & SSM_FLAG_ZOH) == 0 && d->chunk_size == 0 &&
        L >= 256 && L % vw == 0) {
        const int64_t W = d->batch * p->n_cblk;
        const int64_t rounds = W / kSimds, surplus = W - rounds * kSimds;
        const int64_t waves = rounds * kSimds + 2 * surplus;
        const double m0 = static_cast<double>(ceil_div(W, kSimds));
        const double m1 = static_cast<double>(rounds) + ceil_div(2 * surplus, kSimds) / 2.8 * 1.8;
        if (rounds >= 1 && surplus > 0 && waves <= 3 * kSimds && m1 < 0.9 * m0) {
            int64_t k = (L * 10 / 28 + 15) / 16 * 16;
            if (k < 16) k = 16;
            p->split_full = rounds * kSimds;
            p->K = k;
            p->J = 2;
            p->fold = 1;
            const size_t cj = static_cast<size_t>(d->batch) * d->d_inner * 2;
            size_t off = 0;
            p->off_hend = off;
            off += align_up(cj * 16 * sizeof(float));
            p->off_dtsum = off;
            off += align_up(cj * sizeof(float));
            p->off_keep = off;
            off += align_up(static_cast<size_t>(d->batch) * 2 * sizeof(float));
            p->off_flags = off;
            off += align_up(static_cast<size_t>(W) * 2 * sizeof(uint64_t));
            p->bytes = off;
            return SSM_OK;
        }
    }
    int64_t K;
    if (d->chunk_size > 0) {
        K = d->chunk_size;
    } else {
        const int64_t waves = d->batch * p->n_cblk * (p->quad ? 1 : GW);
        K = L;
        if (waves < kEnoughWaves) {
            const int64_t J = (kTargetWaves + waves - 1) / waves;
            int64_t k = (L + J - 1) / J;
            k = (k + 15) / 16 * 16;
            if (k < kMinAutoChunk) k = kMinAutoChunk;
            // chunks this short run as two passes: balance their SIMDs
            if (p->quad && k < kFusedMinChunk) k = quad_auto_chunk(L, waves);
            if (k < L) K = k;
        }
    }
    if (K >= L) K = L;
    p->K = K;
    p->J = (L + K - 1) / K;
    if (p->J > kMaxGridY) return SSM_ERR_UNSUPPORTED;
    if (p->n_cblk * d->batch > static_cast<int64_t>(UINT_MAX)) return SSM_ERR_UNSUPPORTED;
    p->fold = p->J <= kFoldMaxChunks;
    p->fused = fwd && p->quad && p->fold && p->J > 1 && K >= kFusedMinChunk;
    // workspace layout: the chunk operators and, without folding, the chunk
    // start states; rows of G * 16 floats per (batch, channel, chunk)
    size_t off = 0;
    if (p->J > 1) {
        const size_t cj = static_cast<size_t>(d->batch) * d->d_inner * p->J;
        p->off_hend = off;
        off += align_up(cj * G * 16 * sizeof(float));
        p->off_dtsum = off;
        off += align_up(cj * sizeof(float));
        p->off_keep = off;
        off += align_up(static_cast<size_t>(d->batch) * p->J * sizeof(float));
        if (!p->fold) {
            p->off_hstart = off;
            off += align_up(cj * G * 16 * sizeof(float));
        }
        if (p->fused) {
            p->off_flags = off;
            off += align_up(static_cast<size_t>(d->batch) * p->n_cblk * p->J * sizeof(uint64_t));
        }
    }
    p->bytes = off;
    return SSM_OK;
}

bool aligned(const void *p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// Epochs of one-launch scans: unique per launch within the process, and
// seeded from the clock and this object's address so that flags left in
// reused memory by another process or library instance do not match either.
uint64_t next_epoch() {
    static std::atomic<uint64_t> counter{
        (static_cast<uint64_t>(std::chrono::steady_clock::now().time_since_epoch().count()) *
         0x9E3779B97F4A7C15ull) ^
        reinterpret_cast<uintptr_t>(&counter)};
    uint64_t e = counter.fetch_add(1, std::memory_order_relaxed);
    return e != 0 ? e : counter.fetch_add(1, std::memory_order_relaxed);
}

// Backward plan: its own chunks (bwd_auto_chunk, or the caller's chunk
// length), at most 32 of them (each chunk folds its neighbours' operators
// itself), and the workspace of the backward.

struct BwdPlan {
    Plan f;
    int64_t n_tiles = 0;
    // with the forward's checkpoints (no packed sequences): blocks below
    // `split` in every batch row as one chunk, the others in J_s chunks of K_s
    int64_t split = 0, J_s = 0, K_s = 0;
    size_t off_gend = 0, off_bdtsum = 0, off_ckpt = 0, off_dBp = 0, off_dCp = 0, off_dAp = 0,
           off_dDp = 0, off_dbp = 0, bytes = 0;
};

// The backward kernel holds two wavefronts per SIMD (one with ZOH): this many
// run at once on 256 CUs x 4 SIMDs.
constexpr int64_t kBwdSlots = 2048;

// Chunk length of the backward's own plan (chunk_size 0), from the
// wavefronts w = batch x channel blocks of one chunk.  When the chunks of one
// round fit (w <= slots): the most chunks (at most 32, of at least 64 tokens)
// whose J x w wavefronts still run in a single round.  Otherwise: the J that
// minimises rounds x chunk length, ceil(J w / slots) K, with each chunk after
// the first counted as 1% more (its reverse aggregate and fold).  Measured on
// MI355X with the forward checkpoints given: 2 x 1536 channels x 2048 tokens
// (w = 192) 252 us at 11 chunks (2112 wavefronts, a second round of 64),
// 246 us at 10, 281 us at 12; 8 x 5120 channels x 2048 tokens (w = 2560)
// 2945 us in one chunk (1.25 rounds), 2787 us in 2, 2693 us in 4 (5 rounds).
int64_t bwd_auto_chunk(int64_t L, int64_t w, int64_t slots) {
    auto chunk = [&](int64_t J) {
        int64_t k = (L + J - 1) / J;
        k = (k + 15) / 16 * 16;
        return k < L ? k : L;
    };
    if (w <= slots) {
        int64_t J = slots / w;
        if (J > kFoldMaxChunks) J = kFoldMaxChunks;
        if (J > L / kMinAutoChunk) J = L / kMinAutoChunk;
        return J > 1 ? chunk(J) : L;
    }
    int64_t best_k = L;
    double best = 1e300;
    for (int64_t J = 1; J <= kFoldMaxChunks; ++J) {
        const int64_t k = chunk(J);
        if (J > 1 && k < kMinAutoChunk) break;
        const int64_t jr = (L + k - 1) / k;
        const int64_t rounds = (jr * w + slots - 1) / slots;
        const double cost = static_cast<double>(rounds) * k * (1.0 + 0.01 * (jr - 1));
        if (cost < best) { best = cost; best_k = k; }
    }
    return best_k;
}

ssm_status make_bwd_plan(const ssm_desc *d, BwdPlan *p) {
    const ssm_status st = make_plan(d, &p->f, false);
    if (st != SSM_OK) return st;
    if (d->d_state > 16) return SSM_ERR_UNSUPPORTED;
    Plan &f = p->f;
    const int64_t L = d->seqlen;
    if (L == 0 || d->batch * d->d_inner == 0) { p->bytes = 0; return SSM_OK; }
    if (d->chunk_size == 0) {
        const int64_t slots = (d->flags & SSM_FLAG_ZOH) ? kBwdSlots / 2 : kBwdSlots;
        f.K = bwd_auto_chunk(L, d->batch * f.n_cblk, slots);
        f.J = (L + f.K - 1) / f.K;
    }
    if (f.J > kFoldMaxChunks) {
        int64_t k = (L + kFoldMaxChunks - 1) / kFoldMaxChunks;
        k = (k + 15) / 16 * 16;
        f.K = k < L ? k : L;
        f.J = (L + f.K - 1) / f.K;
    }
    f.fold = 1;
    // Split by chunk count, for calls given the forward's checkpoints (no
    // forward chunk operators needed): when the blocks take more than one
    // round of wavefront slots, a whole round of them (the first `split`
    // blocks of every batch row) runs as one chunk and only the rest is cut
    // into chunks, which fill one more round.  The wavefronts then scan as
    // many tokens per SIMD as with every block in chunks, and the reverse
    // chunk aggregates cover the rest alone.
    if (d->chunk_size == 0) {
        const int64_t slots = (d->flags & SSM_FLAG_ZOH) ? kBwdSlots / 2 : kBwdSlots;
        const int64_t w = d->batch * f.n_cblk;
        const int64_t split = slots / d->batch;
        if (w > slots && split >= 1 && split < f.n_cblk) {
            const int64_t rest = d->batch * (f.n_cblk - split);
            int64_t Js = slots / rest;
            if (Js > kFoldMaxChunks) Js = kFoldMaxChunks;
            if (Js > L / kMinAutoChunk) Js = L / kMinAutoChunk;
            if (Js < 1) Js = 1;
            int64_t Ks = (L + Js - 1) / Js;
            Ks = (Ks + 15) / 16 * 16;
            if (Ks > L) Ks = L;
            Js = (L + Ks - 1) / Ks;
            auto cost = [&](int64_t J, int64_t K, int64_t waves) {
                return static_cast<double>((waves + slots - 1) / slots) * K * (1.0 + 0.01 * (J - 1));
            };
            const double c_split = static_cast<double>(L) + cost(Js, Ks, rest * Js);
            const double c_all = cost(f.J, f.K, w * f.J);
            if (Js > 1 && Js <= kFoldMaxChunks && c_split <= c_all) {
                p->split = split; p->J_s = Js; p->K_s = Ks;
            }
        }
    }
    const size_t B = static_cast<size_t>(d->batch), D = static_cast<size_t>(d->d_inner);
    // per-chunk arrays sized for either schedule
    const size_t J = static_cast<size_t>(f.J > p->J_s ? f.J : p->J_s);
    p->n_tiles = (L + ssm::kBwdTile - 1) / ssm::kBwdTile;
    size_t off = 0;
    if (J > 1) {
        f.off_hend = off; off += align_up(B * D * J * 16 * sizeof(float));
        f.off_dtsum = off; off += align_up(B * D * J * sizeof(float));
        f.off_keep = off; off += align_up(B * J * sizeof(float));
        p->off_gend = off; off += align_up(B * D * J * 16 * sizeof(float));
        p->off_bdtsum = off; off += align_up(B * D * J * sizeof(float));
    }
    p->off_ckpt = off; off += align_up(B * D * static_cast<size_t>(p->n_tiles) * 16 * sizeof(float));
    const size_t part = B * static_cast<size_t>(f.n_cblk) * 16 * static_cast<size_t>(L);
    p->off_dBp = off; off += align_up(part * sizeof(float));
    p->off_dCp = off; off += align_up(part * sizeof(float));
    p->off_dAp = off; off += align_up(B * D * J * 16 * sizeof(float));
    p->off_dDp = off; off += align_up(B * D * J * sizeof(float));
    p->off_dbp = off; off += align_up(B * D * J * sizeof(float));
    p->bytes = off;
    return SSM_OK;
}

// Backward with d_state > 16 (ufo.work article, §3.2: the state dimension
// splits into groups that recur independently): the 16-state pass runs once
// per group of 16 states on that group's slices of A, B, C, the start state
// and dlast.  The per-token sums over states add (du, ddelta, dz, d(bias));
// D's terms enter with group 0 alone; dA, dB, dC and dh0 are the groups'
// slices.  No packed sequences or forward checkpoints on this path.
//
// When one group's 16-channel blocks fill under half of the backward's
// wavefront slots, P groups (up to 4) run side by side in one launch, each
// as one chunk: no chunk operators to compute, where one group alone would
// need its sequence cut into chunks to fill the chip.  Each group writes its
// du, ddelta and dz to a workspace slot of its own (no launch reads what
// another wrote: adding in place costs a launch about a fifth more), and
// the slots are summed in group order at the end; this path is taken while
// the slots take at most kMaxGroupSlotBytes.  Otherwise (P = 1) the groups
// run one launch each, group 0 writing du, ddelta and dz and each later one
// adding to them in place.
constexpr size_t kMaxGroupSlotBytes = size_t(8) << 30;
struct BwdGroupPlan {
    ssm_desc sd{};   // the 16-state descriptor of one group
    BwdPlan sub;
    int64_t NG = 0, P = 1;
    // per-slot sizes (bytes; multiples of kAlign) of the P slots of each buffer
    size_t s_sub = 0, s_BC = 0, s_A = 0, s_S = 0, s_dBC = 0, s_db = 0, s_out = 0;
    size_t off_sub = 0, off_B = 0, off_C = 0, off_A = 0, off_h0 = 0, off_dl = 0, off_dA = 0,
           off_dB = 0, off_dC = 0, off_db = 0, off_dh0 = 0, off_du = 0, off_dd = 0, off_dz = 0,
           bytes = 0;
};

ssm_status make_bwd_group_plan(const ssm_desc *d, BwdGroupPlan *p) {
    const ssm_status st = check_desc(d);
    if (st != SSM_OK) return st;
    if (d->d_state <= 16) return SSM_ERR_UNSUPPORTED;
    p->NG = (d->d_state + 15) / 16;
    const size_t B = static_cast<size_t>(d->batch), D = static_cast<size_t>(d->d_inner);
    const size_t L = static_cast<size_t>(d->seqlen);
    const size_t esz = d->io_dtype == SSM_BF16 ? 2 : 4;
    p->sd = *d;
    p->sd.d_state = 16;
    p->sd.workspace = nullptr;
    p->sd.workspace_bytes = 0;
    p->sd.profile_begin = p->sd.profile_end = nullptr;
    // groups side by side: P of them fill at least 3/4 of the wavefront
    // slots, and the groups' du, ddelta and dz slots fit the bound
    const int64_t w = d->batch * ((d->d_inner + 15) / 16);
    const int64_t slots = (d->flags & SSM_FLAG_ZOH) ? kBwdSlots / 2 : kBwdSlots;
    p->P = 1;
    if (d->chunk_size == 0 && w > 0 && L > 0) {
        int64_t P = slots / w;
        if (P > 4) P = 4;
        if (P > p->NG) P = p->NG;
        const size_t out = align_up(B * D * L * sizeof(float));
        if (P >= 2 && 4 * P * w >= 3 * slots &&
            3 * static_cast<size_t>(p->NG) * out <= kMaxGroupSlotBytes)
            p->P = P;
    }
    if (p->P > 1) p->sd.chunk_size = static_cast<int64_t>((L + 15) / 16 * 16);   // one chunk
    ssm_status s2 = make_bwd_plan(&p->sd, &p->sub);
    if (s2 == SSM_OK && p->P > 1 && p->sub.f.J != 1) {
        p->P = 1;
        p->sd.chunk_size = d->chunk_size;
        s2 = make_bwd_plan(&p->sd, &p->sub);
    }
    if (s2 != SSM_OK) return s2;
    const size_t P = static_cast<size_t>(p->P);
    p->s_sub = align_up(p->sub.bytes);
    p->s_BC = align_up(B * 16 * L * esz);
    p->s_A = align_up(D * 16 * sizeof(float));
    p->s_S = align_up(B * D * 16 * sizeof(float));
    p->s_dBC = align_up(B * 16 * L * sizeof(float));
    p->s_db = align_up(D * sizeof(float));
    p->s_out = P > 1 ? align_up(B * D * L * sizeof(float)) : 0;
    const size_t S = P > 1 ? static_cast<size_t>(p->NG) : 0;   // a slot per group
    size_t off = 0;
    auto take = [&](size_t &o, size_t slot) { o = off; off += P * slot; };
    take(p->off_sub, p->s_sub);
    take(p->off_B, p->s_BC);
    take(p->off_C, p->s_BC);
    take(p->off_A, p->s_A);
    take(p->off_h0, p->s_S);
    take(p->off_dl, p->s_S);
    take(p->off_dA, p->s_A);
    take(p->off_dB, p->s_dBC);
    take(p->off_dC, p->s_dBC);
    take(p->off_db, p->s_db);
    take(p->off_dh0, p->s_S);
    auto take_s = [&](size_t &o, size_t slot) { o = off; off += S * slot; };
    take_s(p->off_du, p->s_out);
    take_s(p->off_dd, p->s_out);
    take_s(p->off_dz, p->s_out);
    p->bytes = off;
    return SSM_OK;
}

}  // namespace

namespace {

struct ConvSpec {
    int width = 0;
    int silu = 0;
    const float *weight = nullptr, *bias = nullptr, *state = nullptr;
    void *u_out = nullptr;
};

ssm_status scan_impl(const ssm_desc *desc, const void *u, const ConvSpec &cv, const void *delta,
                     const float *A, const void *B, const void *C, const float *D, const void *z,
                     const float *delta_bias, int softplus_flag, const float *initial_state,
                     const int32_t *cu_seqlens, int64_t n_seqs, void *y, float *last_state,
                     float *ckpt, ssm_stream_t stream) {
    Plan p;
    const bool lean = !cu_seqlens && cv.width == 0;
    ssm_status st = make_plan(desc, &p, true, lean);
    if (st != SSM_OK) return st;
    const hipStream_t s = stream;
    if (cu_seqlens && (desc->batch != 1 || n_seqs < 1)) return SSM_ERR_BAD_SHAPE;
    const int64_t state_rows = cu_seqlens ? n_seqs : desc->batch;
    if (!dims_ok(state_rows, desc->d_inner, desc->d_state)) return SSM_ERR_BAD_SHAPE;
    const int64_t rows = desc->batch * desc->d_inner;
    if (rows == 0) return SSM_OK;
    const size_t esz = desc->io_dtype == SSM_BF16 ? 2 : 4;
    if (!A) return SSM_ERR_NULL_ARG;
    if (cv.width != 0 && (cv.width < 1 || cv.width > SSM_MAX_CONV_WIDTH))
        return SSM_ERR_UNSUPPORTED;
    if (cv.width != 0 && !cv.weight) return SSM_ERR_NULL_ARG;
    if (!aligned(A, 4) || !aligned(D, 4) || !aligned(delta_bias, 4) || !aligned(last_state, 4) ||
        !aligned(initial_state, 4) || !aligned(cu_seqlens, 4) || !aligned(cv.weight, 4) ||
        !aligned(cv.bias, 4) || !aligned(cv.state, 4) || !aligned(cv.u_out, esz))
        return SSM_ERR_MISALIGNED;
    if (desc->seqlen == 0) {
        // every sequence is empty: its final state is its initial state
        if (last_state) {
            const size_t n = static_cast<size_t>(state_rows) * desc->d_inner * desc->d_state;
            const hipError_t e =
                initial_state ? hipMemcpyAsync(last_state, initial_state, n * sizeof(float),
                                               hipMemcpyDeviceToDevice, s)
                              : ssm::launch_fill_zero(last_state, n, s);
            if (e != hipSuccess) return SSM_ERR_HIP;
        }
        return SSM_OK;
    }
    if (!u || !delta || !B || !C || !y) return SSM_ERR_NULL_ARG;
    if (!aligned(u, esz) || !aligned(delta, esz) || !aligned(B, esz) || !aligned(C, esz) ||
        !aligned(y, esz) || !aligned(z, esz))
        return SSM_ERR_MISALIGNED;
    if (ckpt && !p.quad) return SSM_ERR_UNSUPPORTED;
    if (!aligned(ckpt, 16)) return SSM_ERR_MISALIGNED;
    if (p.bytes > 0) {
        if (!desc->workspace || desc->workspace_bytes < p.bytes) return SSM_ERR_WORKSPACE;
        if (!aligned(desc->workspace, 16)) return SSM_ERR_MISALIGNED;
    }
    char *ws = static_cast<char *>(desc->workspace);
    ScanArgs a{};
    a.Bsz = desc->batch; a.D = desc->d_inner; a.N = desc->d_state; a.L = desc->seqlen;
    a.G = p.G; a.K = p.K; a.J = p.J; a.n_cblk = p.n_cblk; a.quad = p.quad;
    a.bf16 = desc->io_dtype == SSM_BF16;
    a.softplus = softplus_flag != 0;
    a.zoh = (desc->flags & SSM_FLAG_ZOH) != 0;
    a.u = u; a.delta = delta; a.z = z; a.B = B; a.C = C; a.y = y;
    a.A = A; a.Dskip = D; a.delta_bias = delta_bias; a.last_state = last_state;
    a.h0 = initial_state; a.cu = cu_seqlens; a.n_seqs = cu_seqlens ? n_seqs : desc->batch;
    a.conv_w = cv.width; a.conv_silu = cv.silu; a.conv_weight = cv.weight;
    a.conv_bias = cv.bias; a.conv_state = cv.state; a.u_out = cv.u_out;
    a.ckpt = ckpt;
    a.n_ck = (desc->seqlen + ssm::kBwdTile - 1) / ssm::kBwdTile;
    if (p.J > 1) {
        a.hend = reinterpret_cast<float *>(ws + p.off_hend);
        a.dtsum = reinterpret_cast<float *>(ws + p.off_dtsum);
        a.keep = reinterpret_cast<float *>(ws + p.off_keep);
        if (!p.fold) a.hstart = reinterpret_cast<float *>(ws + p.off_hstart);
        if (p.fused || p.split_full > 0) {
            a.n_full = p.split_full;
            a.flags = reinterpret_cast<uint64_t *>(ws + p.off_flags);
            a.epoch = next_epoch();
            // a chunk's aggregate pass takes ~0.1 us per token; wait up to
            // 50 us + 0.3 us per token (100 MHz ticks) before computing a
            // missing predecessor operator locally
            const uint64_t ticks = 5000u + 30u * static_cast<uint64_t>(p.K);
            a.spin_ticks = (desc->flags & SSM_FLAG_INDEPENDENT_CHUNKS) ? 0
                           : ticks < kMaxSpinTicks                   ? ticks
                                                                     : kMaxSpinTicks;
            // A captured graph replays this launch with the same epoch: clear
            // the flags ahead of it (a kernel node, not a memset node), so that
            // a replay never reads the operators of the replay before it.
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            if (hipStreamIsCapturing(s, &cs) != hipSuccess) return SSM_ERR_HIP;
            if (cs != hipStreamCaptureStatusNone) {
                // 8-byte flags, cleared as pairs of floats
                const size_t n = static_cast<size_t>(desc->batch) * p.n_cblk * p.J * 2;
                if (ssm::launch_fill_zero(reinterpret_cast<float *>(a.flags), n, s) != hipSuccess)
                    return SSM_ERR_HIP;
            }
        }
    }
    a.ev_begin = static_cast<hipEvent_t>(desc->profile_begin);
    a.ev_end = static_cast<hipEvent_t>(desc->profile_end);
    if (p.tile_ts > 0) {
        a.tile_ts = p.tile_ts;
        return ssm::launch_tscan(a, s) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
    }
    return ssm::launch_scan(a, s) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

// The backward for d_state <= 16 (ssm_scan_bwd_ex's own path).  accumulate:
// du, ddelta and dz are added to what they hold instead of overwritten (the
// later groups of states of bwd_groups); never with packed sequences.
ssm_status bwd_single(const ssm_desc *desc, const void *u, const void *delta, const float *A,
                      const void *B, const void *C, const float *D, const void *z,
                      const float *delta_bias, int softplus_flag, const float *initial_state,
                      const int32_t *cu_seqlens, int64_t n_seqs, const float *ckpt,
                      const void *dy, const float *dlast, float *du, float *ddelta, float *dA,
                      float *dB, float *dC, float *dD, float *dz, float *ddelta_bias, float *dh0,
                      int accumulate, ssm_stream_t stream,
                      const ssm::BwdArgs *side_by_side = nullptr) {
    BwdPlan p;
    ssm_status st = make_bwd_plan(desc, &p);
    if (st != SSM_OK) return st;
    if (cu_seqlens && (desc->batch != 1 || n_seqs < 1)) return SSM_ERR_BAD_SHAPE;
    if (cu_seqlens && accumulate) return SSM_ERR_UNSUPPORTED;
    const int64_t state_rows = cu_seqlens ? n_seqs : desc->batch;
    if (!dims_ok(state_rows, desc->d_inner, desc->d_state)) return SSM_ERR_BAD_SHAPE;
    if (!aligned(cu_seqlens, 4) || !aligned(ckpt, 16)) return SSM_ERR_MISALIGNED;
    const int64_t rows = desc->batch * desc->d_inner;
    if (rows == 0 || desc->seqlen == 0) {
        // no tokens: every gradient of a token is empty; those of the
        // parameters are zero and dh0 = dlast
        const hipStream_t s = stream;
        auto zero = [&](float *ptr, size_t n) {
            return ptr ? ssm::launch_fill_zero(ptr, n, s) : hipSuccess;
        };
        const size_t N = static_cast<size_t>(desc->d_state), Dn = static_cast<size_t>(desc->d_inner);
        hipError_t e = zero(dA, Dn * N);
        if (e == hipSuccess) e = zero(dD, Dn);
        if (e == hipSuccess) e = zero(ddelta_bias, Dn);
        if (e == hipSuccess && dh0) {
            const size_t n = static_cast<size_t>(state_rows) * Dn * N;
            e = dlast ? hipMemcpyAsync(dh0, dlast, n * sizeof(float), hipMemcpyDeviceToDevice, s)
                      : ssm::launch_fill_zero(dh0, n, s);
        }
        return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
    }
    if (!u || !delta || !A || !B || !C || !dy || !du || !ddelta || !dA || !dB || !dC)
        return SSM_ERR_NULL_ARG;
    const size_t esz = desc->io_dtype == SSM_BF16 ? 2 : 4;
    if (!aligned(u, esz) || !aligned(delta, esz) || !aligned(B, esz) || !aligned(C, esz) ||
        !aligned(z, esz) || !aligned(dy, esz) || !aligned(A, 4) || !aligned(D, 4) ||
        !aligned(delta_bias, 4) || !aligned(initial_state, 4) || !aligned(dlast, 4) ||
        !aligned(du, 4) || !aligned(ddelta, 4) || !aligned(dA, 4) || !aligned(dB, 4) ||
        !aligned(dC, 4) || !aligned(dD, 4) || !aligned(dz, 4) || !aligned(ddelta_bias, 4) ||
        !aligned(dh0, 4))
        return SSM_ERR_MISALIGNED;
    if (z && !dz) return SSM_ERR_NULL_ARG;
    if (!desc->workspace || desc->workspace_bytes < p.bytes) return SSM_ERR_WORKSPACE;
    if (!aligned(desc->workspace, 16)) return SSM_ERR_MISALIGNED;
    char *ws = static_cast<char *>(desc->workspace);
    const Plan &f = p.f;
    ScanArgs a{};
    a.Bsz = desc->batch; a.D = desc->d_inner; a.N = desc->d_state; a.L = desc->seqlen;
    a.G = f.G; a.K = f.K; a.J = f.J; a.n_cblk = f.n_cblk; a.quad = f.quad;
    a.bf16 = desc->io_dtype == SSM_BF16;
    a.softplus = softplus_flag != 0;
    a.zoh = (desc->flags & SSM_FLAG_ZOH) != 0;
    a.u = u; a.delta = delta; a.z = z; a.B = B; a.C = C;
    a.A = A; a.Dskip = D; a.delta_bias = delta_bias; a.h0 = initial_state;
    a.cu = cu_seqlens;
    a.n_seqs = state_rows;
    ssm::BwdArgs g{};
    g.accumulate = accumulate;
    g.dy = dy; g.dlast = dlast; g.du = du; g.ddelta = ddelta; g.dz = dz; g.dA = dA; g.dB = dB;
    g.dC = dC; g.dD = dD; g.dbias = ddelta_bias; g.dh0 = dh0; g.n_tiles = p.n_tiles;
    if (f.J > 1 || p.J_s > 1) {
        a.hend = reinterpret_cast<float *>(ws + f.off_hend);
        a.dtsum = reinterpret_cast<float *>(ws + f.off_dtsum);
        a.keep = reinterpret_cast<float *>(ws + f.off_keep);
        g.gend = reinterpret_cast<float *>(ws + p.off_gend);
        g.bdtsum = reinterpret_cast<float *>(ws + p.off_bdtsum);
    }
    // the forward pass's checkpoints (read only), or the workspace's
    g.ckpt = ckpt ? const_cast<float *>(ckpt) : reinterpret_cast<float *>(ws + p.off_ckpt);
    g.ckpt_given = ckpt != nullptr;
    g.dBp = reinterpret_cast<float *>(ws + p.off_dBp);
    g.dCp = reinterpret_cast<float *>(ws + p.off_dCp);
    g.dAp = reinterpret_cast<float *>(ws + p.off_dAp);
    g.dDp = reinterpret_cast<float *>(ws + p.off_dDp);
    g.dbp = reinterpret_cast<float *>(ws + p.off_dbp);
    if (ckpt && !cu_seqlens && !side_by_side && p.split > 0) {
        // the whole-round blocks in one chunk, the rest in J_s chunks
        a.J = p.J_s; a.K = p.K_s;
        g.split = p.split;
    }
    if (side_by_side) {   // groups of states side by side: one chunk each
        if (f.J != 1 || cu_seqlens || ckpt) return SSM_ERR_UNSUPPORTED;
        const ssm::BwdArgs &x = *side_by_side;
        g.gz = x.gz;
        g.gs_A = x.gs_A; g.gs_BC = x.gs_BC; g.gs_S = x.gs_S; g.gs_out = x.gs_out;
        g.gs_ws = x.gs_ws; g.gs_dBC = x.gs_dBC; g.gs_db = x.gs_db;
    }
    return ssm::launch_bwd(a, g, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status bwd_groups(const ssm_desc *desc, const void *u, const void *delta, const float *A,
                      const void *B, const void *C, const float *D, const void *z,
                      const float *delta_bias, int softplus_flag, const float *initial_state,
                      const void *dy, const float *dlast, float *du, float *ddelta, float *dA,
                      float *dB, float *dC, float *dD, float *dz, float *ddelta_bias, float *dh0,
                      ssm_stream_t stream) {
    BwdGroupPlan p;
    const ssm_status st = make_bwd_group_plan(desc, &p);
    if (st != SSM_OK) return st;
    const int64_t Bn = desc->batch, Dn = desc->d_inner, N = desc->d_state, L = desc->seqlen;
    const hipStream_t s = stream;
    if (Bn * Dn == 0 || L == 0) {
        // no tokens: as the 16-state pass, over all N states
        auto zero = [&](float *ptr, size_t n) {
            return ptr ? ssm::launch_fill_zero(ptr, n, s) : hipSuccess;
        };
        hipError_t e = zero(dA, static_cast<size_t>(Dn * N));
        if (e == hipSuccess) e = zero(dD, static_cast<size_t>(Dn));
        if (e == hipSuccess) e = zero(ddelta_bias, static_cast<size_t>(Dn));
        if (e == hipSuccess && dh0) {
            const size_t n = static_cast<size_t>(Bn * Dn * N);
            e = dlast ? hipMemcpyAsync(dh0, dlast, n * sizeof(float), hipMemcpyDeviceToDevice, s)
                      : ssm::launch_fill_zero(dh0, n, s);
        }
        return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
    }
    if (!u || !delta || !A || !B || !C || !dy || !du || !ddelta || !dA || !dB || !dC)
        return SSM_ERR_NULL_ARG;
    if (z && !dz) return SSM_ERR_NULL_ARG;
    const size_t esz = desc->io_dtype == SSM_BF16 ? 2 : 4;
    if (!aligned(B, esz) || !aligned(C, esz) || !aligned(A, 4) || !aligned(initial_state, 4) ||
        !aligned(dlast, 4) || !aligned(dA, 4) || !aligned(dB, 4) || !aligned(dC, 4) ||
        !aligned(dh0, 4) || !aligned(du, 4) || !aligned(ddelta, 4) || !aligned(dz, 4) ||
        !aligned(ddelta_bias, 4))
        return SSM_ERR_MISALIGNED;
    if (!desc->workspace || desc->workspace_bytes < p.bytes) return SSM_ERR_WORKSPACE;
    if (!aligned(desc->workspace, 16)) return SSM_ERR_MISALIGNED;
    char *ws = static_cast<char *>(desc->workspace);
    auto at = [&](size_t off) { return reinterpret_cast<float *>(ws + off); };
    ssm_desc sd = p.sd;
    sd.workspace = ws + p.off_sub;
    sd.workspace_bytes = p.P * p.s_sub;
    void *Bg = ws + p.off_B, *Cg = ws + p.off_C;
    float *Ag = at(p.off_A), *h0g = initial_state ? at(p.off_h0) : nullptr;
    float *dlg = dlast ? at(p.off_dl) : nullptr;
    float *dAg = at(p.off_dA), *dBg = at(p.off_dB), *dCg = at(p.off_dC);
    float *dh0g = dh0 ? at(p.off_dh0) : nullptr;
    const int ie = static_cast<int>(esz);
    // groups g .. g + np - 1 into (out of) slots 0 .. np - 1, one launch per buffer
    const int64_t e_BC = static_cast<int64_t>(p.s_BC / esz), e_A = static_cast<int64_t>(p.s_A / 4),
                  e_S = static_cast<int64_t>(p.s_S / 4), e_dBC = static_cast<int64_t>(p.s_dBC / 4);
    auto gather = [&](int64_t g, int np) {
        const int64_t n0 = 16 * g;
        hipError_t e = ssm::launch_gather_rows(Bg, B, Bn, N, n0, L, ie, s, np, e_BC);
        if (e == hipSuccess) e = ssm::launch_gather_rows(Cg, C, Bn, N, n0, L, ie, s, np, e_BC);
        if (e == hipSuccess) e = ssm::launch_gather_cols(Ag, A, Dn, N, n0, s, np, e_A);
        if (e == hipSuccess && h0g)
            e = ssm::launch_gather_cols(h0g, initial_state, Bn * Dn, N, n0, s, np, e_S);
        if (e == hipSuccess && dlg)
            e = ssm::launch_gather_cols(dlg, dlast, Bn * Dn, N, n0, s, np, e_S);
        return e;
    };
    auto scatter = [&](int64_t g, int np) {
        const int64_t n0 = 16 * g;
        hipError_t e = ssm::launch_scatter_cols(dA, dAg, Dn, N, n0, s, np, e_A);
        if (e == hipSuccess) e = ssm::launch_scatter_rows(dB, dBg, Bn, N, n0, L, s, np, e_dBC);
        if (e == hipSuccess) e = ssm::launch_scatter_rows(dC, dCg, Bn, N, n0, L, s, np, e_dBC);
        if (e == hipSuccess && dh0g)
            e = ssm::launch_scatter_cols(dh0, dh0g, Bn * Dn, N, n0, s, np, e_S);
        return e;
    };
    if (p.P == 1) {
        for (int64_t g = 0; g < p.NG; ++g) {
            hipError_t e = gather(g, 1);
            if (e != hipSuccess) return SSM_ERR_HIP;
            // group 0 writes du, ddelta, dz and d(bias); each later group adds
            // its share to du, ddelta and dz in place (old + new, in group
            // order) and its d(bias) through a small buffer
            const bool first = g == 0;
            float *db_o = ddelta_bias ? (first ? ddelta_bias : at(p.off_db)) : nullptr;
            const ssm_status sst = bwd_single(
                &sd, u, delta, Ag, Bg, Cg, first ? D : nullptr, z, delta_bias, softplus_flag, h0g,
                nullptr, 0, nullptr, dy, dlg, du, ddelta, dAg, dBg, dCg, first ? dD : nullptr,
                z ? dz : nullptr, db_o, dh0g, first ? 0 : 1, stream);
            if (sst != SSM_OK) return sst;
            if (!first && db_o) e = ssm::launch_accumulate(ddelta_bias, db_o, Dn, s);
            if (e == hipSuccess) e = scatter(g, 1);
            if (e != hipSuccess) return SSM_ERR_HIP;
        }
        return SSM_OK;
    }
    // P groups side by side per launch
    ssm::BwdArgs x{};
    x.gs_A = static_cast<int64_t>(p.s_A / sizeof(float));
    x.gs_BC = static_cast<int64_t>(p.s_BC);
    x.gs_S = static_cast<int64_t>(p.s_S / sizeof(float));
    x.gs_out = static_cast<int64_t>(p.s_out / sizeof(float));
    x.gs_ws = static_cast<int64_t>(p.s_sub);
    x.gs_dBC = static_cast<int64_t>(p.s_dBC / sizeof(float));
    x.gs_db = static_cast<int64_t>(p.s_db / sizeof(float));
    float *du_s = at(p.off_du), *dd_s = at(p.off_dd), *dz_s = z ? at(p.off_dz) : nullptr;
    float *db_s = ddelta_bias ? at(p.off_db) : nullptr;
    hipError_t e = ddelta_bias ? ssm::launch_fill_zero(ddelta_bias, static_cast<size_t>(Dn), s)
                               : hipSuccess;
    if (e != hipSuccess) return SSM_ERR_HIP;
    for (int64_t g0 = 0; g0 < p.NG; g0 += p.P) {
        const int np = static_cast<int>(p.NG - g0 < p.P ? p.NG - g0 : p.P);
        e = gather(g0, np);
        if (e != hipSuccess) return SSM_ERR_HIP;
        x.gz = np;
        const bool first = g0 == 0;
        const int64_t s0 = g0 * x.gs_out;   // groups g0 .. g0 + np - 1: their own slots
        const ssm_status sst = bwd_single(
            &sd, u, delta, Ag, Bg, Cg, first ? D : nullptr, z, delta_bias, softplus_flag, h0g,
            nullptr, 0, nullptr, dy, dlg, du_s + s0, dd_s + s0, dAg, dBg, dCg,
            first ? dD : nullptr, dz_s ? dz_s + s0 : nullptr, db_s, dh0g, 0, stream, &x);
        if (sst != SSM_OK) return sst;
        e = scatter(g0, np);
        if (e == hipSuccess && db_s)   // d(bias) in group order
            e = ssm::launch_accumulate(ddelta_bias, db_s, Dn, s, np, x.gs_db);
        if (e != hipSuccess) return SSM_ERR_HIP;
    }
    // du, ddelta, dz: the groups' slots summed in group order
    const int ng = static_cast<int>(p.NG);
    const int64_t n = Bn * Dn * L;
    e = ssm::launch_sum_slots(du, du_s, ng, x.gs_out, n, s);
    if (e == hipSuccess) e = ssm::launch_sum_slots(ddelta, dd_s, ng, x.gs_out, n, s);
    if (e == hipSuccess && dz_s) e = ssm::launch_sum_slots(dz, dz_s, ng, x.gs_out, n, s);
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

// ---------------------------------------------------------------- no-allocation scratch
// The workspace of ssm_scan_fwd_noalloc.  Each GPU that the library runs on
// holds its own copy of this array.  In host code its name is only a
// host-side stand-in: the device address of each GPU's copy is looked up
// with hipGetSymbolAddress, once per device with that device current, and
// only that address is ever passed on.
static __device__ __align__(256) unsigned char scratch[SSM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 256;
std::atomic<void *> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// The device address of the scratch array of the GPU that `stream` runs on
// (the current device for the null stream).
ssm_status scratch_address(hipStream_t stream, void **out) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return SSM_ERR_HIP;
    int dev = cur;
    if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return SSM_ERR_HIP;
    if (dev < 0 || dev >= kMaxScratchDevices) return SSM_ERR_UNSUPPORTED;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (dev != cur && hipSetDevice(dev) != hipSuccess) return SSM_ERR_HIP;
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (dev != cur && hipSetDevice(cur) != hipSuccess) return SSM_ERR_HIP;
            if (e != hipSuccess || !p) return SSM_ERR_HIP;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return SSM_OK;
}

}  // namespace

extern "C" {

size_t ssm_scan_workspace_bytes(const ssm_desc *desc) {
    // enough for every forward entry point: calls with packed sequences or
    // the fused convolution may plan chunks where a plain call runs the
    // in-wave scan (none) or the balanced serial walks (their own)
    Plan plain, other;
    if (make_plan(desc, &plain, true, true) != SSM_OK) return 0;
    if (make_plan(desc, &other, true, false) != SSM_OK) return 0;
    return plain.bytes > other.bytes ? plain.bytes : other.bytes;
}

int64_t ssm_scan_chunk_size(const ssm_desc *desc) {
    Plan p;
    return make_plan(desc, &p) == SSM_OK ? p.K : -1;
}

const char *ssm_scan_plan(const ssm_desc *desc) {
    Plan p;
    if (make_plan(desc, &p) != SSM_OK) return "invalid";
    if (p.tile_ts == 16) return "in-wave scan: chunks of 256 tokens in sequence, 16 segments of 16";
    if (p.tile_ts == 8) return "in-wave scan: chunks of 128 tokens in sequence, 16 segments of 8";
    if (p.split_full > 0) return "one chunk, the blocks past the last whole round in two chunks (one launch)";
    if (p.J <= 1) return "one chunk";
    if (p.fused) return "one launch: chunk aggregates, fold and y";
    if (p.fold) return "two passes: chunk aggregates, then y with the fold";
    return "two passes and the carry kernel";
}

ssm_status ssm_scan_fwd_ex(const ssm_desc *desc, const void *u, const void *delta, const float *A,
                           const void *B, const void *C, const float *D, const void *z,
                           const float *delta_bias, int softplus_flag, const float *initial_state,
                           const int32_t *cu_seqlens, int64_t n_seqs, void *y, float *last_state,
                           ssm_stream_t stream) {
    return scan_impl(desc, u, ConvSpec{}, delta, A, B, C, D, z, delta_bias, softplus_flag,
                     initial_state, cu_seqlens, n_seqs, y, last_state, nullptr, stream);
}

ssm_status ssm_scan_fwd_conv(const ssm_desc *desc, const void *x, const float *conv_weight,
                             const float *conv_bias, int conv_width, int conv_silu,
                             const float *conv_state, const void *delta, const float *A,
                             const void *B, const void *C, const float *D, const void *z,
                             const float *delta_bias, int softplus_flag,
                             const float *initial_state, const int32_t *cu_seqlens,
                             int64_t n_seqs, void *y, float *last_state, void *u_out,
                             ssm_stream_t stream) {
    if (conv_width < 1 || conv_width > SSM_MAX_CONV_WIDTH) {
        if (!desc) return SSM_ERR_NULL_ARG;
        return SSM_ERR_UNSUPPORTED;
    }
    ConvSpec cv;
    cv.width = conv_width; cv.silu = conv_silu != 0; cv.weight = conv_weight;
    cv.bias = conv_bias; cv.state = conv_state; cv.u_out = u_out;
    return scan_impl(desc, x, cv, delta, A, B, C, D, z, delta_bias, softplus_flag, initial_state,
                     cu_seqlens, n_seqs, y, last_state, nullptr, stream);
}

ssm_status ssm_scan_fwd_ckpt(const ssm_desc *desc, const void *u, const void *delta,
                             const float *A, const void *B, const void *C, const float *D,
                             const void *z, const float *delta_bias, int softplus_flag,
                             const float *initial_state, const int32_t *cu_seqlens,
                             int64_t n_seqs, void *y, float *last_state, float *ckpt,
                             ssm_stream_t stream) {
    if (!ckpt) return SSM_ERR_NULL_ARG;
    return scan_impl(desc, u, ConvSpec{}, delta, A, B, C, D, z, delta_bias, softplus_flag,
                     initial_state, cu_seqlens, n_seqs, y, last_state, ckpt, stream);
}

size_t ssm_scan_ckpt_bytes(const ssm_desc *desc) {
    Plan p;
    if (make_plan(desc, &p) != SSM_OK || !p.quad) return 0;
    const size_t tiles = static_cast<size_t>((desc->seqlen + ssm::kBwdTile - 1) / ssm::kBwdTile);
    return static_cast<size_t>(desc->batch) * static_cast<size_t>(desc->d_inner) * tiles * 16 *
           sizeof(float);
}

ssm_status ssm_scan_fwd(const ssm_desc *desc, const void *u, const void *delta, const float *A,
                        const void *B, const void *C, const float *D, const void *z,
                        const float *delta_bias, int softplus_flag, void *y, float *last_state,
                        ssm_stream_t stream) {
    return ssm_scan_fwd_ex(desc, u, delta, A, B, C, D, z, delta_bias, softplus_flag, nullptr,
                           nullptr, 0, y, last_state, stream);
}

ssm_status ssm_scan_fwd_noalloc(const ssm_desc *desc, const void *u, const void *delta,
                                const float *A, const void *B, const void *C, const float *D,
                                const void *z, const float *delta_bias, int softplus_flag,
                                void *y, float *last_state, ssm_stream_t stream) {
    if (!desc) return SSM_ERR_NULL_ARG;
    ssm_desc d = *desc;
    d.workspace = nullptr;
    d.workspace_bytes = 0;
    Plan p;
    const ssm_status st = make_plan(&d, &p);   // the plan of a plain call
    if (st != SSM_OK) return st;
    if (p.bytes > SSM_NOALLOC_SCRATCH_BYTES) return SSM_ERR_WORKSPACE;
    if (p.bytes > 0) {
        void *ws = nullptr;
        const ssm_status s2 = scratch_address(stream, &ws);
        if (s2 != SSM_OK) return s2;
        d.workspace = ws;
        d.workspace_bytes = SSM_NOALLOC_SCRATCH_BYTES;
    }
    return ssm_scan_fwd(&d, u, delta, A, B, C, D, z, delta_bias, softplus_flag, y, last_state,
                        stream);
}

ssm_status ssm_state_update(const ssm_desc *desc, float *state, const void *u, const void *delta,
                            const float *A, const void *B, const void *C, const float *D,
                            const void *z, void *y, ssm_stream_t stream) {
    if (!desc) return SSM_ERR_NULL_ARG;
    if (desc->batch < 0 || desc->d_inner < 0) return SSM_ERR_BAD_SHAPE;
    if (desc->d_state < 1 || desc->d_state > SSM_MAX_D_STATE) return SSM_ERR_UNSUPPORTED;
    if (desc->io_dtype != SSM_F32 && desc->io_dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
    if ((desc->flags & ~kKnownFlags) != 0 || desc->reserved != 0) return SSM_ERR_UNSUPPORTED;
    if (!dims_ok(desc->batch, desc->d_inner, desc->d_state)) return SSM_ERR_BAD_SHAPE;
    if (desc->batch * desc->d_inner == 0) return SSM_OK;
    if (!state || !u || !delta || !A || !B || !C || !y) return SSM_ERR_NULL_ARG;
    const size_t esz = desc->io_dtype == SSM_BF16 ? 2 : 4;
    if (!aligned(state, 4) || !aligned(A, 4) || !aligned(D, 4) || !aligned(u, esz) ||
        !aligned(delta, esz) || !aligned(B, esz) || !aligned(C, esz) || !aligned(z, esz) ||
        !aligned(y, esz))
        return SSM_ERR_MISALIGNED;
    ssm::UpdateArgs a{};
    a.Bsz = desc->batch; a.D = desc->d_inner; a.N = desc->d_state;
    a.bf16 = desc->io_dtype == SSM_BF16;
    a.zoh = (desc->flags & SSM_FLAG_ZOH) != 0;
    a.state = state; a.u = u; a.delta = delta; a.z = z; a.B = B; a.C = C; a.y = y;
    a.A = A; a.Dskip = D;
    return ssm::launch_update(a, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

const char *ssm_scan_bwd_plan(const ssm_desc *desc, int with_ckpt) {
    if (desc && desc->d_state > 16) {
        BwdGroupPlan p;
        if (make_bwd_group_plan(desc, &p) != SSM_OK || with_ckpt) return "invalid";
        return p.P > 1 ? "groups of 16 states side by side, one chunk each"
                       : "groups of 16 states one per launch";
    }
    BwdPlan p;
    if (make_bwd_plan(desc, &p) != SSM_OK) return "invalid";
    if (with_ckpt && p.split > 0) return "the blocks of a whole round in one chunk, the rest in chunks";
    return p.f.J <= 1 ? "one chunk" : "chunks joined by reverse chunk aggregates";
}

size_t ssm_scan_bwd_workspace_bytes(const ssm_desc *desc) {
    if (desc && desc->d_state > 16) {
        BwdGroupPlan p;
        return make_bwd_group_plan(desc, &p) == SSM_OK ? p.bytes : 0;
    }
    BwdPlan p;
    return make_bwd_plan(desc, &p) == SSM_OK ? p.bytes : 0;
}

ssm_status ssm_scan_bwd_ex(const ssm_desc *desc, const void *u, const void *delta,
                           const float *A, const void *B, const void *C, const float *D,
                           const void *z, const float *delta_bias, int softplus_flag,
                           const float *initial_state, const int32_t *cu_seqlens, int64_t n_seqs,
                           const float *ckpt, const void *dy, const float *dlast, float *du,
                           float *ddelta, float *dA, float *dB, float *dC, float *dD, float *dz,
                           float *ddelta_bias, float *dh0, ssm_stream_t stream) {
    if (desc && desc->d_state > 16) {
        if (cu_seqlens || ckpt) return SSM_ERR_UNSUPPORTED;
        return bwd_groups(desc, u, delta, A, B, C, D, z, delta_bias, softplus_flag,
                          initial_state, dy, dlast, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias,
                          dh0, stream);
    }
    return bwd_single(desc, u, delta, A, B, C, D, z, delta_bias, softplus_flag, initial_state,
                      cu_seqlens, n_seqs, ckpt, dy, dlast, du, ddelta, dA, dB, dC, dD, dz,
                      ddelta_bias, dh0, 0, stream);
}

ssm_status ssm_scan_bwd(const ssm_desc *desc, const void *u, const void *delta, const float *A,
                        const void *B, const void *C, const float *D, const void *z,
                        const float *delta_bias, int softplus_flag, const float *initial_state,
                        const void *dy, const float *dlast, float *du, float *ddelta, float *dA,
                        float *dB, float *dC, float *dD, float *dz, float *ddelta_bias,
                        float *dh0, ssm_stream_t stream) {
    return ssm_scan_bwd_ex(desc, u, delta, A, B, C, D, z, delta_bias, softplus_flag,
                           initial_state, nullptr, 0, nullptr, dy, dlast, du, ddelta, dA, dB, dC,
                           dD, dz, ddelta_bias, dh0, stream);
}

const char *ssm_status_string(int status) {
    switch (status) {
        case SSM_OK: return "SSM_OK";
        case SSM_ERR_NULL_ARG: return "SSM_ERR_NULL_ARG: a required pointer is NULL";
        case SSM_ERR_BAD_SHAPE: return "SSM_ERR_BAD_SHAPE: invalid dimension or chunk_size";
        case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED: d_state or io_dtype not supported";
        case SSM_ERR_MISALIGNED: return "SSM_ERR_MISALIGNED: pointer not aligned to its element";
        case SSM_ERR_WORKSPACE: return "SSM_ERR_WORKSPACE: workspace missing or too small";
        case SSM_ERR_HIP: return "SSM_ERR_HIP: kernel launch failed";
        default: return "unknown status";
    }
}

int ssm_version(void) { return 500; }

}  // extern "C"
