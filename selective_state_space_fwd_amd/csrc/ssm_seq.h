// ssm_seq.h -- sequence bookkeeping shared by the forward and backward
// kernels: where the state starts over (batch rows, or packed sequences of
// a cu_seqlens table) and the start states.
#pragma once

#include "ssm_common.h"
#include "ssm_launch.h"

namespace ssm {

// Where the state starts over: at token 0 of every batch row or, with packed
// sequences (ufo.work article, §4.2), at the first token of every sequence of
// the cu_seqlens table.  All values here are uniform across a workgroup.
// Offsets are clamped into [0, L], so any table keeps every access in bounds.
__device__ __forceinline__ int64_t cu_at(const ScanArgs &a, int64_t i) {
    const int64_t v = a.cu[i];
    return v < 0 ? 0 : (v > a.L ? a.L : v);
}

// The sequence that token t belongs to: the last s with cu[s] <= t (empty
// sequences that start at t come before it and are skipped).
__device__ __forceinline__ int64_t seq_of(const ScanArgs &a, int64_t t) {
    int64_t lo = 0, hi = a.n_seqs - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (cu_at(a, mid) <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

struct SeqPos {
    int64_t s;        // sequence: the batch row when sequences are not packed
    int64_t end;      // its end, the next token where the state starts over
    bool reset;       // token t starts the sequence
};

template <bool EXT>
__device__ __forceinline__ SeqPos seq_pos(const ScanArgs &a, int64_t b, int64_t t) {
    SeqPos p;
    if (EXT && a.cu) {
        p.s = seq_of(a, t);
        p.end = cu_at(a, p.s + 1);
        p.reset = cu_at(a, p.s) == t;
    } else {
        p.s = b;
        p.end = a.L;
        p.reset = t == 0;
    }
    return p;
}

// States n0 .. n0 + S - 1 of channel dcl in row s of a (rows, d_inner, N)
// state array p (zero when p is null, for states n >= N and padded channels).
template <int S>
__device__ __forceinline__ void load_state_row(const float *p, const ScanArgs &a, int64_t s,
                                               int64_t dcl, bool lane_ok, int n0, float (&h)[S]) {
#pragma unroll
    for (int k = 0; k < S; ++k) {
        const int n = n0 + k;
        const float v = p ? p[(s * a.D + dcl) * a.N + (n < a.N ? n : a.N - 1)] : 0.0f;
        h[k] = (lane_ok && n < a.N) ? v : 0.0f;
    }
}

// Start state of sequence s for states n0 .. n0 + S - 1 of channel d (zero
// when there is no initial state, for states n >= N and for padded channels).
template <int S>
__device__ __forceinline__ void load_start_state(const ScanArgs &a, int64_t s, int64_t dcl,
                                                 bool lane_ok, int n0, float (&h)[S]) {
    load_state_row<S>(a.h0, a, s, dcl, lane_ok, n0, h);
}

// Writes states n0 .. n0 + S - 1 of channel d into row s of p (if not null).
template <int S>
__device__ __forceinline__ void store_state_row(float *p, const ScanArgs &a, int64_t s, int64_t d,
                                                bool lane_ok, int n0, const float (&h)[S]) {
    if (!p || !lane_ok) return;
    float *row = p + (s * a.D + d) * a.N;
#pragma unroll
    for (int k = 0; k < S; ++k)
        if (n0 + k < a.N) row[n0 + k] = h[k];
}

// Sequence marks of the n <= 32 tokens t0 .. t0 + n - 1 (packed sequences):
// bit i of the result is set when token t0 + i starts a sequence, bit i of
// *last when it is the last token of its sequence (the next token starts one,
// or it is the row's last token).  Tokens past the row have no marks.
__device__ __forceinline__ uint32_t seq_marks(const ScanArgs &a, int64_t t0, int n,
                                              uint32_t *last) {
    uint32_t st = 0, ls = 0;
    const int64_t t1 = t0 + n;
    // the boundaries p in [t0, t1]: sequence starts cu[s], s >= seq_of(t0), and the row end
    for (int64_t s = seq_of(a, t0); s <= a.n_seqs; ++s) {
        const int64_t p = s < a.n_seqs ? cu_at(a, s) : a.L;
        if (p > t1) break;
        if (p >= t0 && p < t1 && p < a.L) st |= 1u << (p - t0);
        if (p > t0) ls |= 1u << (p - 1 - t0);
    }
    if (a.L > t0 && a.L <= t1) ls |= 1u << (a.L - 1 - t0);
    *last = ls;
    return st;
}

}  // namespace ssm
