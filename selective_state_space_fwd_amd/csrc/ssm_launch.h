// ssm_launch.h -- host-side launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssm {

// Everything a prefill scan launch needs; built and validated by ssm_api.
struct ScanArgs {
    int64_t Bsz, D, N, L;       // batch, d_inner, d_state, seqlen
    int G;                      // groups of 16 states in a padded state row (power of two):
                                // 1 for quad_kernel, 2 x its wavefronts for group_kernel
    int64_t K, J, n_cblk;       // chunk length, chunk count, 16-channel blocks per batch row
    int quad;                   // 1: d_state <= 16 path (quad_kernel), else group_kernel
    int bf16;                   // io dtype
    int softplus;
    int zoh;                    // zero-order-hold input term
    const void *u, *delta, *z, *B, *C;
    void *y;
    const float *A, *Dskip, *delta_bias;
    float *last_state;          // (rows, d_inner, N): rows = batch, or n_seqs when packed
    const float *h0;            // initial states, same rows as last_state, or null (zeros)
    const int32_t *cu;          // packed sequences: n_seqs + 1 token offsets (batch == 1), or null
    int64_t n_seqs;
    // optional depthwise causal conv1d ahead of the scan: u then holds its
    // input x, and the scan input is silu(conv(x) + bias)
    int conv_w;                 // taps, 0 = no convolution
    int conv_silu;
    const float *conv_weight;   // (d_inner, conv_w)
    const float *conv_bias;     // (d_inner) or null
    const float *conv_state;    // (rows, d_inner, conv_w - 1): inputs before each sequence, or null
    void *u_out;                // optional: the scan input (batch, d_inner, L), io dtype
    // workspace views
    float *hend;                // (batch, d_inner, J, G*16) chunk end states from zero
    float *dtsum;               // (batch, d_inner, J) sum of step sizes per chunk
    float *keep;                // (batch, J) 1: the chunk keeps its incoming state, 0: it
                                // starts a sequence somewhere, so its operator's decay is 0
    float *hstart;              // (batch, d_inner, J, G*16) chunk start states
    // one-launch chunked scan (quad path, 1 < J <= 32): per (batch, channel
    // block, chunk) publication flags, this launch's epoch, and how long (in
    // ticks of the 100 MHz real-time clock) a chunk waits for the chunks
    // before it before computing their operators itself; null flags: two passes
    uint64_t *flags;
    uint64_t epoch;
    uint64_t spin_ticks;
    // optional (quad path): the pass that writes y also writes the state
    // entering every kBwdTile-token tile, (batch, d_inner, n_ck, 16), for
    // the backward pass
    float *ckpt;
    int64_t n_ck;
    hipEvent_t ev_begin, ev_end;  // optional: start of the first dispatch, end of the last
    // > 0: 16-channel blocks 0 .. n_full-1 walk the whole sequence and each
    // later block runs as two chunks, tokens 0 .. K-1 and K .. L-1, on two
    // wavefronts (quad_split_kernel; J = 2 workspace layout, flags, epoch)
    int64_t n_full;
    // > 0: the in-wave scan with segments of tile_ts tokens (tscan_kernel),
    // whose launcher sets n_cblk to its own channel blocks
    int tile_ts;
};

// Tokens per backward tile: the spacing of the state checkpoints.
#ifndef SSM_BWD_TILE
#define SSM_BWD_TILE 8
#endif
constexpr int kBwdTile = SSM_BWD_TILE;
static_assert(kBwdTile == 4 || kBwdTile == 8, "backward tile of 4 or 8 tokens");

// Backward pass (d_state <= 16): upstream gradients, outputs and its own
// workspace views; the forward quantities come from a ScanArgs.
struct BwdArgs {
    const void *dy;             // (batch, d_inner, L) io dtype
    const float *dlast;         // (batch, d_inner, N) or null
    float *du, *ddelta, *dz;    // (batch, d_inner, L); dz only with a gate
    float *dA;                  // (d_inner, N)
    float *dB, *dC;             // (batch, N, L)
    float *dD, *dbias;          // (d_inner) or null
    float *dh0;                 // (batch, d_inner, N) or null
    int64_t n_tiles;            // backward tiles per row (checkpoints)
    int ckpt_given;             // ckpt holds the forward pass's checkpoints: no forward sweep
    // workspace views
    float *ckpt;                // (batch, d_inner, n_tiles, 16) state entering each tile
    float *gend;                // (batch, d_inner, J, 16) gradient leaving each chunk to its left, from zero
    float *bdtsum;              // (batch, d_inner, J) sum of step sizes (reverse order)
    float *dBp, *dCp;           // (batch, n_cblk, 16, L) per 16-channel block
    float *dAp;                 // (batch, d_inner, J, 16)
    float *dDp, *dbp;           // (batch, d_inner, J)
    int accumulate;             // du, ddelta, dz: add to what they hold (lean and ZOH instances)
    // Groups of 16 states side by side (d_state > 16): gz groups in one launch,
    // group blockIdx.z; every pointer above is group 0's, and group z's lies
    // z strides further (one chunk only: no chunk operators).  D's terms and
    // dD belong to group 0 alone.
    int gz;                     // 0 or 1: one group
    int64_t gs_A;               // floats: A (d_inner, 16) and dA
    int64_t gs_BC;              // bytes: B and C (batch, 16, L)
    int64_t gs_S;               // floats: start state, dlast, dh0 (batch, d_inner, 16)
    int64_t gs_out;             // floats: du, ddelta, dz (batch, d_inner, L)
    int64_t gs_ws;              // bytes: the workspace views (ckpt, dBp, dCp, dAp, dDp, dbp)
    int64_t gs_dBC;             // floats: dB and dC (batch, 16, L)
    int64_t gs_db;              // floats: dbias (d_inner)
    // Blocks split by chunk count (forward checkpoints given, no packed
    // sequences): in every batch row, channel blocks below `split` run as one
    // chunk, the others in J chunks.  A launch covers blocks cblk0 .. cblk0 +
    // ncb - 1 of every row (ncb 0: all of them); the per-chunk arrays (gend,
    // bdtsum, dAp, dDp, dbp) hold Jl chunks per channel (0: J).
    int64_t split, cblk0, ncb, Jl;
};

hipError_t launch_bwd(const ScanArgs &a, const BwdArgs &g, hipStream_t s);

// P groups of 16 states (n0 .. n0 + 15, then n0 + 16 .. n0 + 31, ...) out of
// N, for the backward with d_state > 16; group p's slice lies p slots (of
// `slot` elements) into the gathered buffer.  Rows: dst (R, 16, L) <-> src
// (R, N, L); columns: dst (R, 16) <-> src (R, N).  Gathers zero-fill states
// n >= N; scatters skip them.
hipError_t launch_gather_rows(void *dst, const void *src, int64_t R, int64_t N, int64_t n0,
                              int64_t L, int esz, hipStream_t s, int P = 1, int64_t slot = 0);
hipError_t launch_gather_cols(float *dst, const float *src, int64_t R, int64_t N, int64_t n0,
                              hipStream_t s, int P = 1, int64_t slot = 0);
hipError_t launch_scatter_rows(float *dst, const float *src, int64_t R, int64_t N, int64_t n0,
                               int64_t L, hipStream_t s, int P = 1, int64_t slot = 0);
hipError_t launch_scatter_cols(float *dst, const float *src, int64_t R, int64_t N, int64_t n0,
                               hipStream_t s, int P = 1, int64_t slot = 0);
// dst[i] += src[i], then += src[i + slot], ... (P terms, in that order), i < n
hipError_t launch_accumulate(float *dst, const float *src, int64_t n, hipStream_t s, int P = 1,
                             int64_t slot = 0);
// dst[i] = src[i] + src[i + stride] + ... + src[i + (P - 1) stride], added in
// that order, i < n
hipError_t launch_sum_slots(float *dst, const float *src, int P, int64_t stride, int64_t n,
                            hipStream_t s);

struct UpdateArgs {
    int64_t Bsz, D, N;
    int bf16;
    int zoh;
    float *state;
    const void *u, *delta, *z, *B, *C;
    void *y;
    const float *A, *Dskip;
};

hipError_t launch_scan(const ScanArgs &a, hipStream_t s);
// The in-wave scan (d_state <= 16, no packed sequences or convolution).
hipError_t launch_tscan(const ScanArgs &a, hipStream_t s);
// Only the forward chunk-aggregate pass (chunks 0 .. J-2), d_state <= 16.
hipError_t launch_scan_agg(const ScanArgs &a, hipStream_t s);
hipError_t launch_update(const UpdateArgs &a, hipStream_t s);
hipError_t launch_fill_zero(float *p, size_t n, hipStream_t s);

}  // namespace ssm
