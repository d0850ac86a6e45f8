// libpalimpsa: the Palimpsa dual-state recurrence on MI355X (gfx950).
//
// Recurrence ("Learning to Remember, Learn, and Forget in Attention-Based
// Models", slides frames "Palimpsa updates content and importance together"
// and "Natural parameters expose two affine scans", Eq. (5), App. A.12),
// per head, value channel i, key channel j, token t:
//
//   alpha_t = exp(-A dt_t),  c_t = (1 - alpha_t) I_prior
//   I_t  = alpha_t I_{t-1} + c_t + beta_t[i] k_t[j]^2
//   M_t  = alpha_t M_{t-1} + (beta_t[i] v_t[i]) k_t[j]        (M = I . mu)
//   y_t[i] = sum_j (M_t / I_t)[i, j] q_t[j]                   (read after the write)
//
// Chunked forward (palimpsa_fwd_chunked)
// --------------------------------------
// The readout divides by a per-token, per-entry precision, so no step is a
// dense contraction: the kernel is bound by the FP32 vector ALU, not by HBM
// (a few hundred GB/s) and not by the matrix cores.  Each state entry costs
// four FMA/MUL pairs' worth of VALU work per token: 6 VALU instructions and
// one v_rcp_f32.  Everything else is arranged so that those instructions are
// nearly all the SIMDs issue:
//
//  * The state (M, I) never leaves VGPRs between the first and the last
//    token: one workgroup owns 16 value rows of one head for the whole
//    sequence, so no inter-chunk state goes to HBM.
//  * Lane layout: a wave owns 4 value rows; 16 lanes share a row and each
//    owns DK/16 key columns (8 at d_k = 128).  Each lane keeps its partial
//    readout of 16 consecutive tokens in registers; one transposing DPP
//    reduction then leaves token g's row sum in lane g (2.8 VALU ops per
//    token instead of a 4-step all-reduce per token), and each lane stores
//    one y value per 16 tokens.
//  * Per chunk of C tokens the workgroup stages, once, the per-column
//    operands k, k^2, q (float32), the per-row pair (beta, beta*v) and the
//    per-token gate (alpha, c) in LDS; bf16 is widened once here, not per
//    lane.  Staging is double-buffered: the global loads of chunk n+1 are in
//    flight while chunk n is computed, and one barrier separates chunks.
//  * Column operands are read from LDS as 128-bit vectors with the 16 lanes
//    of a row covering 256 contiguous bytes (conflict-free); the 4 rows of a
//    wave read the same addresses (broadcast).
//  * blockIdx -> (head, row block) is remapped so the row blocks of one head
//    run on one XCD and share k/q through that XCD's L2.
//
// Decode step (palimpsa_step)
// ---------------------------
// One token over a state held as (mu, I): 16 bytes of state are read and
// written per entry, so the kernel streams HBM with 128-bit non-temporal
// accesses; the arithmetic is a few percent of the memory time.
//
// Precision: all arithmetic is float32; bf16 inputs are widened exactly and
// bf16 outputs are rounded to nearest even.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "palimpsa.h"

#define PALIMPSA_VERSION 100  // 0.1.0

// The no-allocation forward's scratch (see device_scratch below): 64 MiB per
// GPU, enough for every time split the library chooses by itself on MI355X.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

typedef __bf16 bf16_t;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

template <typename T> struct io;
// bits()/from_bits(): a scalar kept in its raw bits between a prefetch and its
// use, so that the widening (and the wait for the load) happens at the use
// and not where the load is issued; bits 0 is 0.0 in both types.
template <> struct io<float> {
    __device__ static inline float to_f32(float x) { return x; }
    __device__ static inline float from_f32(float x) { return x; }
    __device__ static inline uint32_t bits(float x) { return __float_as_uint(x); }
    __device__ static inline float from_bits(uint32_t b) { return __uint_as_float(b); }
};
template <> struct io<bf16_t> {
    __device__ static inline float to_f32(bf16_t x) { return (float)x; }
    __device__ static inline bf16_t from_f32(float x) { return (bf16_t)x; }  // RNE
    __device__ static inline uint32_t bits(bf16_t x) { return __builtin_bit_cast(uint16_t, x); }
    __device__ static inline float from_bits(uint32_t b) { return __uint_as_float(b << 16); }
};

// Widen a 16-byte packet of T to float32 values.
template <typename T> struct packet;
template <> struct packet<float> {
    static constexpr int kN = 4;
    __device__ static inline void widen(const uint4 &p, float *out) {
        out[0] = __uint_as_float(p.x); out[1] = __uint_as_float(p.y);
        out[2] = __uint_as_float(p.z); out[3] = __uint_as_float(p.w);
    }
};
template <> struct packet<bf16_t> {
    static constexpr int kN = 8;
    __device__ static inline void widen(const uint4 &p, float *out) {
        const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};

// Sum over the 16 lanes of a DPP row; every lane receives the total.
__device__ inline float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));  // row_half_mirror
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));  // row_mirror
    return x;
}

// The gate of Eq. (9): alpha = exp(-A dt) and c = (1 - alpha) I_prior, with
// 1 - alpha taken as -expm1(-A dt) so that it keeps full relative accuracy
// when A dt is small.
__device__ inline float2 gate(float A, float dt, float Ip) {
    const float x = -A * dt;
    return make_float2(expf(x), -expm1f(x) * Ip);
}

// ---------------------------------------------------------------------------
// chunked forward
// ---------------------------------------------------------------------------

struct FwdArgs {
    const void *q, *k, *v, *beta, *dt;
    const float *A, *Ip, *mu0, *I0;
    void *y;
    float *muT, *IT;
    int B, T, H, dv;
    int nwg;           // launched workgroups
    int xcd_remap;     // 1: remap so one head's row blocks share an XCD
    int nwg_seg;       // workgroups per time segment: B * H * dv / 16
    int seg_len;       // tokens per time segment (a multiple of the chunk)
    int nseg;          // time segments (1: no split)
    float *ws;         // segment summaries, see SegWs
    float *ck;         // backward checkpoints (kCheckpoint mode, training forward), see bwd_kernel
    int nck;           // checkpoints per sequence: ceil(T / kCkI)
    int vstar;         // 1: v holds beta . v (the write itself)
    int frozen;        // checkpoint pass of the frozen-importance backward: M_0 = I_prior mu0
};

// Workspace of a time-split forward: for each of the first nseg-1 segments,
// its affine summary from a zero state, laid out as M_loc [nseg-1][B*H][dv][dk],
// then Ibar_loc (same shape); then a copy of the caller's start state
// (mu0, I0), [B*H][dv][dk] each; then the decay product P [nseg-1][B*H].
// The replay pass starts every segment from the copy, never from mu0/I0
// themselves: its last segment may overwrite those (muT aliasing mu0, IT
// aliasing I0) while other segments of the same rows have not started yet.
struct SegWs {
    float *M, *Ib, *mu0, *I0, *P;
    size_t per_seg;    // B * H * dv * dk
    __device__ SegWs(float *ws, int nseg, size_t bh, int dv, int dk)
        : per_seg(bh * dv * dk) {
        M = ws;
        Ib = ws + (size_t)(nseg - 1) * per_seg;
        mu0 = Ib + (size_t)(nseg - 1) * per_seg;
        I0 = mu0 + per_seg;
        P = I0 + per_seg;
    }
};

constexpr int kWaves = 4;                 // waves per workgroup (one per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 4;
constexpr int kRowsPerWG = kRowsPerWave * kWaves;   // 16 value rows per workgroup
constexpr int kLanesPerRow = 16;
constexpr int kGroup = 16;                // tokens per transposing reduction (= lanes per row)
constexpr int kSB = 8;                    // tokens per backward sub-block (staging and reverse walk)
constexpr int kCkI = 2 * kSB;             // tokens between checkpoints of the diagonal backward

// LDS floats per staged token: k, k^2, q columns + (beta, beta*v) per row + gate.
template <int DK> struct Stage {
    static constexpr int kColFloats = 3 * DK;
    static constexpr int kRowFloats = 2 * kRowsPerWG;
    static constexpr int kTokFloats = kColFloats + kRowFloats + 2;
};

template <int DK, int C>
constexpr size_t fwd_lds_bytes() { return (size_t)2 * C * Stage<DK>::kTokFloats * sizeof(float); }

// Staging of one chunk of C tokens into an LDS buffer.
//
// Every thread loads and widens k/q packets (16 bytes each); the (v, beta)
// packet pairs start at wave 1, the gate's alpha at wave 2 and its c at wave
// 3, so no wave carries all the extras into the barrier.  Addresses are a per-chunk base
// (uniform) plus a per-thread 32-bit element offset.  Tokens past the end of
// the sequence are staged as neutral updates (k = q = 0, beta = 0, dt = 0, so
// alpha = 1 and c = 0): they leave (M, I) bit-identical and their y is not
// stored, so the last chunk runs the same code as the others.  Without q
// (WITHQ false, for the time-split summary pass) only k is staged.
template <int DK, int C, typename TIn, bool WITHQ>
struct Stager {
    static constexpr int kPerPkt = packet<TIn>::kN;            // elements per 16 B
    static constexpr int kColPkts = DK / kPerPkt;              // packets per k (or q) row
    static constexpr int kHalf = C * kColPkts;                 // k packets per chunk (= q packets)
    static constexpr int kKQ = (WITHQ ? 2 : 1) * kHalf;        // the summary pass needs no q
    static constexpr int kKQPerThread = (kKQ + kThreads - 1) / kThreads;
    static constexpr bool kSplit = kHalf % kThreads == 0;      // packet u is all-k or all-q
    static constexpr int kRowPkts = kRowsPerWG / kPerPkt;      // packets per v (or beta) row slice
    static constexpr int kVB = C * kRowPkts;                   // (v, beta) packet pairs per chunk
    static_assert(kVB <= kThreads, "one (v, beta) pair per thread at most");
    static_assert(C <= kThreads, "one gate per thread at most");

    uint4 kq[kKQPerThread];
    uint4 vv, bb;
    uint32_t dtv = 0, dtc = 0;   // raw bits (io<TIn>::bits) until the commit

    __device__ static inline int vb_slot(int tid) { return (tid + kThreads - 64) % kThreads; }
    __device__ static inline int gate_slot(int tid) { return (tid + kThreads - 128) % kThreads; }
    __device__ static inline int c_slot(int tid) { return (tid + kThreads - 192) % kThreads; }
    __device__ static inline bool is_q(int u, int p) { return kSplit ? (u >= kHalf / kThreads) : (p >= kHalf); }

    // Chunk bases point at token t0 of this (b, h): k/q at [.., DK], v/beta at
    // the workgroup's first row, dt at the token.  `left` = T - t0 tokens remain.
    __device__ inline void load(const TIn *kb, const TIn *qb, const TIn *vb, const TIn *bb_,
                                const TIn *db, int left, int H, int dv, int tid) {
#pragma unroll
        for (int u = 0; u < kKQPerThread; ++u) {
            const int p = tid + u * kThreads;
            if (kKQ % kThreads == 0 || p < kKQ) {
                const bool q = is_q(u, p);
                const int pp = q ? p - kHalf : p;
                const int tt = pp / kColPkts;
                const uint32_t off = (uint32_t)tt * (uint32_t)(H * DK) + (pp % kColPkts) * kPerPkt;
                kq[u] = make_uint4(0, 0, 0, 0);
                if (tt < left) kq[u] = *(const uint4 *)((q ? qb : kb) + off);
            }
        }
        const int pv = vb_slot(tid);
        if (pv < kVB) {
            const int tt = pv / kRowPkts;
            const uint32_t off = (uint32_t)tt * (uint32_t)(H * dv) + (pv % kRowPkts) * kPerPkt;
            vv = make_uint4(0, 0, 0, 0);
            bb = make_uint4(0, 0, 0, 0);
            if (tt < left) {
                vv = *(const uint4 *)(vb + off);
                bb = *(const uint4 *)(bb_ + off);
            }
        }
        const int pg = gate_slot(tid);
        if (pg < C) {
            dtv = 0;
            if (pg < left) dtv = io<TIn>::bits(db[(uint32_t)pg * (uint32_t)H]);
        }
        const int pc = c_slot(tid);
        if (pc < C) {
            dtc = 0;
            if (pc < left) dtc = io<TIn>::bits(db[(uint32_t)pc * (uint32_t)H]);
        }
    }

    // Widen and write the loaded chunk to one LDS buffer.  With vstar the v
    // packets already hold beta . v.
    __device__ inline void commit(float *buf, float A, float Ip, int tid, bool vstar) const {
        float *cols = buf;
        float *rows = buf + C * Stage<DK>::kColFloats;
        float *gates = rows + C * Stage<DK>::kRowFloats;
#pragma unroll
        for (int u = 0; u < kKQPerThread; ++u) {
            const int p = tid + u * kThreads;
            if (kKQ % kThreads == 0 || p < kKQ) {
                const bool q = is_q(u, p);
                const int pp = q ? p - kHalf : p;
                const int tt = pp / kColPkts;
                const int off = (pp % kColPkts) * kPerPkt;
                float x[kPerPkt];
                packet<TIn>::widen(kq[u], x);
                float *dst = cols + tt * Stage<DK>::kColFloats + off;
                if (!q) {   // k and k^2
#pragma unroll
                    for (int e = 0; e < kPerPkt; e += 4) {
                        *(float4 *)(dst + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
                        *(float4 *)(dst + DK + e) = make_float4(x[e] * x[e], x[e + 1] * x[e + 1],
                                                                x[e + 2] * x[e + 2], x[e + 3] * x[e + 3]);
                    }
                } else {    // q
#pragma unroll
                    for (int e = 0; e < kPerPkt; e += 4)
                        *(float4 *)(dst + 2 * DK + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
                }
            }
        }
        const int pv = vb_slot(tid);
        if (pv < kVB) {
            const int tt = pv / kRowPkts;
            const int off = (pv % kRowPkts) * kPerPkt;
            float xv[kPerPkt], xb[kPerPkt];
            packet<TIn>::widen(vv, xv);
            packet<TIn>::widen(bb, xb);
            float *dst = rows + tt * Stage<DK>::kRowFloats + 2 * off;
#pragma unroll
            for (int e = 0; e < kPerPkt; e += 2)
                *(float4 *)(dst + 2 * e) = make_float4(xb[e], vstar ? xv[e] : xb[e] * xv[e], xb[e + 1],
                                                       vstar ? xv[e + 1] : xb[e + 1] * xv[e + 1]);
        }
        // alpha on wave 2 and c = (1 - alpha) I_prior on wave 3 (the gate of Eq. (9))
        const int pg = gate_slot(tid);
        if (pg < C)
            gates[2 * pg] = expf(-A * io<TIn>::from_bits(dtv));
        const int pc = c_slot(tid);
        if (pc < C)
            gates[2 * pc + 1] = -expm1f(-A * io<TIn>::from_bits(dtc)) * Ip;
    }
};

template <int DK>
struct LaneTile {
    static constexpr int kCols = DK / kLanesPerRow;          // key columns per lane
    static constexpr int kVec = kCols < 4 ? kCols : 4;       // floats per LDS vector read
    static constexpr int kNVec = kCols / kVec;
    // column of entry (m, e) for lane g of its row: vectors interleaved so that
    // the 16 lanes of a row read one contiguous 16*kVec-float span per m.
    __device__ static inline int col(int g, int m, int e) { return kVec * g + kLanesPerRow * kVec * m + e; }
};

template <int V> struct vecf;
template <> struct vecf<4> {
    __device__ static inline void ld(const float *p, float *o) {
        const float4 x = *(const float4 *)p; o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    }
    __device__ static inline void st(float *p, const float *o) { *(float4 *)p = make_float4(o[0], o[1], o[2], o[3]); }
};
template <> struct vecf<2> {
    __device__ static inline void ld(const float *p, float *o) {
        const float2 x = *(const float2 *)p; o[0] = x.x; o[1] = x.y;
    }
    __device__ static inline void st(float *p, const float *o) { *(float2 *)p = make_float2(o[0], o[1]); }
};

// Transposing reduction over the 16 lanes g of a DPP row: lane g holds 16
// partial sums x[0..15] (one per token of a group) and returns the row-wide
// sum of x[g].  Four exchange stages; in each, a lane keeps half of its
// values, sends the other half to its partner, and adds what it receives.
// Partners: l^15 (row_mirror), l^7 within each half-row (row_half_mirror),
// l^2 and l^1 (quad permutations).  The four XOR masks span all 16 lanes, and
// the half a lane keeps is chosen by lane bits 3, 2, 1, 0, so lane g ends
// with token 8 b3 + 4 b2 + 2 b1 + b0 = g.  45 VALU ops for 16 tokens.
template <int CTRL>
__device__ inline float dpp_from(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ inline float row16_transpose_sum(const float (&x)[16], int g) {
    const bool b3 = g & 8, b2 = g & 4, b1 = g & 2, b0 = g & 1;
    float s1[8], s2[4], s3[2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        s1[i] = (b3 ? x[i + 8] : x[i]) + dpp_from<0x140>(b3 ? x[i] : x[i + 8]);       // row_mirror
#pragma unroll
    for (int i = 0; i < 4; ++i)
        s2[i] = (b2 ? s1[i + 4] : s1[i]) + dpp_from<0x141>(b2 ? s1[i] : s1[i + 4]);   // row_half_mirror
#pragma unroll
    for (int i = 0; i < 2; ++i)
        s3[i] = (b1 ? s2[i + 2] : s2[i]) + dpp_from<0x4E>(b1 ? s2[i] : s2[i + 2]);    // quad_perm [2,3,0,1]
    return (b0 ? s3[1] : s3[0]) + dpp_from<0xB1>(b0 ? s3[0] : s3[1]);                 // quad_perm [1,0,3,2]
}

// A workgroup's checkpoint block: the lane's values (M[0, N), I[0, N)),
// N = DK / 16 in {2, 4, 8}, as 2N/4 float4s, float4 i of thread tid at
// blk + 4 (i * kThreads + tid), so each access instruction covers 1 KiB of
// contiguous memory.  Written once and read once much later: non-temporal.
template <int N>
__device__ inline void store_pair(float *blk, int tid, const float *M, const float *I) {
    float v[2 * N];
#pragma unroll
    for (int i = 0; i < N; ++i) { v[i] = M[i]; v[N + i] = I[i]; }
#pragma unroll
    for (int i = 0; i < 2 * N; i += 4)
        __builtin_nontemporal_store(f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]},
                                    (f32x4 *)(blk + 4 * ((i / 4) * kThreads + tid)));
}
template <int N>
__device__ inline void load_pair(const float *blk, int tid, float *M, float *I) {
    float v[2 * N];
#pragma unroll
    for (int i = 0; i < 2 * N; i += 4) {
        const f32x4 x = __builtin_nontemporal_load((const f32x4 *)(blk + 4 * ((i / 4) * kThreads + tid)));
        v[i] = x[0]; v[i + 1] = x[1]; v[i + 2] = x[2]; v[i + 3] = x[3];
    }
#pragma unroll
    for (int i = 0; i < N; ++i) { M[i] = v[i]; I[i] = v[N + i]; }
}

// Marks N values as used at this point (see BwdStager::ready).
template <int N>
__device__ inline void regs_ready(const float *x) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" ::"v"(x[i]));
}

// The same layout in LDS (a thread's private slots; every access instruction
// covers 1 KiB of consecutive banks).
template <int N>
__device__ inline void lds_store_pair(float *blk, int tid, const float *M, const float *I) {
    float v[2 * N];
#pragma unroll
    for (int i = 0; i < N; ++i) { v[i] = M[i]; v[N + i] = I[i]; }
#pragma unroll
    for (int i = 0; i < 2 * N; i += 4)
        *(float4 *)(blk + 4 * ((i / 4) * kThreads + tid)) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
}
template <int N>
__device__ inline void lds_load_pair(const float *blk, int tid, float *M, float *I) {
    float v[2 * N];
#pragma unroll
    for (int i = 0; i < 2 * N; i += 4) {
        const float4 x = *(const float4 *)(blk + 4 * ((i / 4) * kThreads + tid));
        v[i] = x.x; v[i + 1] = x.y; v[i + 2] = x.z; v[i + 3] = x.w;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) { M[i] = v[i]; I[i] = v[N + i]; }
}

// The per-token hot loop over one staged chunk.  Per token and lane: for each
// of the lane's DK/16 state entries 6 VALU ops and one v_rcp_f32; the lane's
// partial of y_t goes to a register.  Every 16 tokens one transposing
// reduction leaves y for token g in lane g, which stores it if the token is
// inside the sequence (`left` = tokens remaining from the chunk start).
//
// With a prior per state entry (IPE) the gate's c is staged as 1 - alpha and
// scaled by the lane's prior ipe[s]: one more VALU op per entry and token.
//
// With CKPT (the training forward, C = kCkI = 16) the state before the
// chunk's first token is also stored at the block ck, as the backward's
// checkpoint pass would store it.
template <int DK, int C, typename TOut, bool IPE, bool CKPT>
__device__ inline void compute_chunk(const float *buf, int left, float *M, float *I,
                                     int row_local, int g, TOut *yrow, size_t ystride, const float *ipe,
                                     float *ck = nullptr) {
    using LT = LaneTile<DK>;
    static_assert(C % kGroup == 0, "chunk must be a multiple of 16 tokens");
    static_assert(!CKPT || (C == kCkI && kGroup == kCkI), "checkpointing forward runs chunk 16");
    const float *cbase = buf + LT::col(g, 0, 0);
    const float *rbase = buf + C * Stage<DK>::kColFloats + 2 * row_local;
    // The gate address is the same in every lane; holding it in a VGPR (the
    // empty asm hides its uniformity) lets every gate read be one ds_read_b64
    // with an immediate offset instead of a per-token SGPR-to-VGPR move.
    int goff = C * (Stage<DK>::kColFloats + Stage<DK>::kRowFloats);
    asm volatile("" : "+v"(goff));
    const float *gbase = buf + goff;
#pragma unroll 1
    for (int grp = 0; grp < C / kGroup; ++grp) {
        const float *cg = cbase + grp * kGroup * Stage<DK>::kColFloats;
        const float *rg = rbase + grp * kGroup * Stage<DK>::kRowFloats;
        const float *gg = gbase + grp * kGroup * 2;
        float part[kGroup];
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            if (CKPT && u == 0) store_pair<LT::kCols>(ck, threadIdx.x, M, I);
            const float2 gc = *(const float2 *)(gg + 2 * u);                          // alpha, c
            const float2 rb = *(const float2 *)(rg + u * Stage<DK>::kRowFloats);      // beta, beta*v
            const float *ct = cg + u * Stage<DK>::kColFloats;
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < LT::kNVec; ++m) {
                float kk[LT::kVec], k2[LT::kVec], qq[LT::kVec];
                const int c0 = kLanesPerRow * LT::kVec * m;
                vecf<LT::kVec>::ld(ct + c0, kk);
                vecf<LT::kVec>::ld(ct + DK + c0, k2);
                vecf<LT::kVec>::ld(ct + 2 * DK + c0, qq);
#pragma unroll
                for (int e = 0; e < LT::kVec; ++e) {
                    const int s = m * LT::kVec + e;
                    const float w = fmaf(rb.x, k2[e], IPE ? gc.y * ipe[s] : gc.y);   // c + beta_i k_j^2
                    I[s] = fmaf(gc.x, I[s], w);                     // importance
                    M[s] = fmaf(gc.x, M[s], rb.y * kk[e]);          // natural content
                    const float r = __builtin_amdgcn_rcpf(I[s]);
                    acc = fmaf(M[s] * r, qq[e], acc);               // mu_ij q_j
                }
            }
            part[u] = acc;
        }
        const float yv = row16_transpose_sum(part, g);
        const int tt = grp * kGroup + g;
        if (tt < left)
            yrow[(size_t)tt * ystride] = io<TOut>::from_f32(yv);
    }
}

// Checkpoint pass of the backward over one staged chunk: the forward update
// without readout (the same 4 VALU ops per entry and token as the replay,
// so the states are bit-identical to the forward's), storing (M, I) before
// every kCkI-th token of the sequence: the workgroup's block for the
// checkpoint before token kCkI s is at ckp + s * ck_stride.
template <int DK, int C, bool IPE>
__device__ inline void ckpt_chunk(const float *buf, float *M, float *I, int row_local, int g,
                                  float *ckp, size_t ck_stride, int t0, int ntok, const float *ipe) {
    using LT = LaneTile<DK>;
    static_assert(C % kCkI == 0, "chunk must hold whole checkpoint intervals");
    const float *cbase = buf + LT::col(g, 0, 0);
    const float *rbase = buf + C * Stage<DK>::kColFloats + 2 * row_local;
    int goff = C * (Stage<DK>::kColFloats + Stage<DK>::kRowFloats);
    asm volatile("" : "+v"(goff));
    const float *gbase = buf + goff;
    // rolled over 8-token halves: unrolling a whole interval raises the
    // register count (and lowers the occupancy) without saving any work
#pragma unroll 1
    for (int sb = 0; sb < C / kSB; ++sb) {
        if (sb % 2 == 0 && t0 + sb * kSB < ntok) {
            store_pair<LT::kCols>(ckp + (size_t)((t0 + sb * kSB) / kCkI) * ck_stride, threadIdx.x, M, I);
        }
#pragma unroll
        for (int u0 = 0; u0 < kSB; ++u0) {
            const int u = sb * kSB + u0;
            const float2 gc = *(const float2 *)(gbase + 2 * u);
            const float2 rb = *(const float2 *)(rbase + u * Stage<DK>::kRowFloats);
            const float *ct = cbase + u * Stage<DK>::kColFloats;
#pragma unroll
            for (int m = 0; m < LT::kNVec; ++m) {
                float kk[LT::kVec], k2[LT::kVec];
                const int c0 = kLanesPerRow * LT::kVec * m;
                vecf<LT::kVec>::ld(ct + c0, kk);
                vecf<LT::kVec>::ld(ct + DK + c0, k2);
#pragma unroll
                for (int e = 0; e < LT::kVec; ++e) {
                    const int s = m * LT::kVec + e;
                    const float w = fmaf(rb.x, k2[e], IPE ? gc.y * ipe[s] : gc.y);
                    I[s] = fmaf(gc.x, I[s], w);
                    M[s] = fmaf(gc.x, M[s], rb.y * kk[e]);
                }
            }
        }
    }
}

enum FwdMode { kReplay = 0, kCheckpoint = 2 };

// One launch of the chunked forward.
//
// kReplay: every (head, row block, segment) runs its tokens with the readout.
// Segment 0 starts from (mu0, I0); segment s > 0 starts from the fold of the
// summaries of segments 0..s-1 (M = P M + M_loc, Ibar = P Ibar + Ibar_loc, the
// composition of the affine scans).  The last segment writes (muT, IT).
// Without a split (nseg = 1) this is the whole sequence in one pass.
//
// kCheckpoint (the backward's first pass; nseg = 1): the sequence from
// (mu0, I0) without readout, storing (M, I) before every kCkI-th token.
//
// (The summaries of a split come from summary_mfma_kernel.)
template <int DK, int C, typename TIn, typename TOut, int MODE, bool IPE, bool CKPT = false>
__global__ __launch_bounds__(kThreads) void fwd_chunked_kernel(FwdArgs a) {
    using LT = LaneTile<DK>;
    extern __shared__ float lds[];
    float *buf0 = lds;
    float *buf1 = lds + C * Stage<DK>::kTokFloats;

    // workgroup -> (segment, head, row block), keeping one head's row blocks
    // of a segment on one XCD
    const int rb_per_head = a.dv / kRowsPerWG;
    int wg = blockIdx.x;
    if (a.xcd_remap) {
        const int per_xcd = a.nwg / 8;
        wg = (wg % 8) * per_xcd + wg / 8;
    }
    const int seg = wg / a.nwg_seg;
    wg -= seg * a.nwg_seg;
    const int bh = wg / rb_per_head;
    const int row0 = (wg % rb_per_head) * kRowsPerWG;
    const int b = bh / a.H, h = bh % a.H;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane & (kLanesPerRow - 1);
    const int row_local = wave * kRowsPerWave + (lane >> 4);
    const int row = row0 + row_local;

    // prior: one per head, or (IPE) one per state entry [H, dv, dk]; with IPE
    // the staged c is 1 - alpha and Ip is 1
    const float A = a.A[h], Ip = IPE ? 1.f : a.Ip[h];
    const int t_begin = seg * a.seg_len;
    const int t_end = min(a.T, t_begin + a.seg_len);

    // start state: M = I0 . mu0, I = I0 (or M = 0, I = I_prior), then the
    // earlier segments' summaries folded in
    float M[LT::kCols], I[LT::kCols];
    const size_t srow = ((size_t)bh * a.dv + row) * DK;
    float ipe[IPE ? LT::kCols : 1];
    if (IPE) {
        const float *ip = a.Ip + ((size_t)h * a.dv + row) * DK;
#pragma unroll
        for (int m = 0; m < LT::kNVec; ++m) vecf<LT::kVec>::ld(ip + LT::col(g, m, 0), ipe + m * LT::kVec);
    }
    {
        if (a.mu0) {
            // a split replay reads the summary pass's copy (see SegWs)
            const float *mu0 = a.mu0, *I0 = a.I0;
            if (MODE == kReplay && a.nseg > 1) {
                const SegWs w(a.ws, a.nseg, (size_t)a.B * a.H, a.dv, DK);
                mu0 = w.mu0;
                I0 = w.I0;
            }
#pragma unroll
            for (int m = 0; m < LT::kNVec; ++m) {
                float mu[LT::kVec], ii[LT::kVec];
                vecf<LT::kVec>::ld(mu0 + srow + LT::col(g, m, 0), mu);
                if (a.frozen) {
#pragma unroll
                    for (int e = 0; e < LT::kVec; ++e) ii[e] = Ip;
                } else {
                    vecf<LT::kVec>::ld(I0 + srow + LT::col(g, m, 0), ii);
                }
#pragma unroll
                for (int e = 0; e < LT::kVec; ++e) {
                    I[m * LT::kVec + e] = ii[e];
                    M[m * LT::kVec + e] = ii[e] * mu[e];
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < LT::kCols; ++s) { I[s] = IPE ? ipe[s] : Ip; M[s] = 0.f; }
        }
        if (seg > 0) {
            const SegWs w(a.ws, a.nseg, (size_t)a.B * a.H, a.dv, DK);
#pragma unroll
            for (int s = 0; s < LT::kCols; ++s) I[s] -= IPE ? ipe[s] : Ip;   // Ibar
            for (int sp = 0; sp < seg; ++sp) {
                const float P = w.P[(size_t)sp * a.B * a.H + bh];
#pragma unroll
                for (int m = 0; m < LT::kNVec; ++m) {
                    float ml[LT::kVec], il[LT::kVec];
                    vecf<LT::kVec>::ld(w.M + sp * w.per_seg + srow + LT::col(g, m, 0), ml);
                    vecf<LT::kVec>::ld(w.Ib + sp * w.per_seg + srow + LT::col(g, m, 0), il);
#pragma unroll
                    for (int e = 0; e < LT::kVec; ++e) {
                        M[m * LT::kVec + e] = fmaf(P, M[m * LT::kVec + e], ml[e]);
                        I[m * LT::kVec + e] = fmaf(P, I[m * LT::kVec + e], il[e]);
                    }
                }
            }
#pragma unroll
            for (int s = 0; s < LT::kCols; ++s) I[s] += IPE ? ipe[s] : Ip;
        }
    }

    // per-sequence bases (token t_begin of this (b, h)) and per-token strides
    const size_t seq = ((size_t)b * a.T + t_begin) * a.H + h;   // row of (b, t_begin, h) in [B, T, H]
    const TIn *kseq = (const TIn *)a.k + seq * DK;
    const TIn *qseq = (const TIn *)a.q + seq * DK;
    const TIn *vseq = (const TIn *)a.v + seq * a.dv + row0;
    const TIn *bseq = (const TIn *)a.beta + seq * a.dv + row0;
    const TIn *dseq = (const TIn *)a.dt + seq;
    const size_t kq_tok = (size_t)a.H * DK, vb_tok = (size_t)a.H * a.dv;
    const size_t ystride = (size_t)a.H * a.dv;
    TOut *ybase = MODE == kReplay ? (TOut *)a.y + seq * a.dv + row : nullptr;

    const int ntok = t_end - t_begin;
    const int nchunks = (ntok + C - 1) / C;
    // checkpoints: [B*H][nck][row block][thread][2 DK/16] floats
    const size_t ck_stride = (size_t)rb_per_head * kThreads * 2 * LT::kCols;
    float *ckp = (MODE == kCheckpoint || CKPT)
                     ? a.ck + ((size_t)bh * a.nck * rb_per_head + row0 / kRowsPerWG) * (kThreads * 2 * LT::kCols)
                     : nullptr;
    Stager<DK, C, TIn, MODE == kReplay> st;
    if (nchunks > 0) {
        st.load(kseq, qseq, vseq, bseq, dseq, ntok, a.H, a.dv, tid);
        st.commit(buf0, A, Ip, tid, a.vstar);
        __syncthreads();
    }
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C;
        const bool more = c + 1 < nchunks;
        if (more) {
            const size_t tn = (size_t)(t0 + C);
            st.load(kseq + tn * kq_tok, qseq + tn * kq_tok, vseq + tn * vb_tok, bseq + tn * vb_tok,
                    dseq + tn * a.H, ntok - (t0 + C), a.H, a.dv, tid);
        }
        const float *cur = (c & 1) ? buf1 : buf0;
        if (MODE == kReplay)
            compute_chunk<DK, C, TOut, IPE, CKPT>(
                cur, ntok - t0, M, I, row_local, g, ybase + (size_t)t0 * ystride, ystride, ipe,
                CKPT ? ckp + (size_t)(t0 / kCkI) * ck_stride : nullptr);
        else
            ckpt_chunk<DK, C, IPE>(cur, M, I, row_local, g, ckp, ck_stride, t0, ntok, ipe);
        if (more) st.commit((c & 1) ? buf0 : buf1, A, Ip, tid, a.vstar);
        __syncthreads();
    }

    if (MODE == kCheckpoint) return;

    // final state (last segment only): mu = M / I (correctly rounded division), I
    if (a.muT && seg == a.nseg - 1) {
#pragma unroll
        for (int m = 0; m < LT::kNVec; ++m) {
            float mu[LT::kVec], ii[LT::kVec];
            if (a.T == 0 && a.mu0) {
                vecf<LT::kVec>::ld(a.mu0 + srow + LT::col(g, m, 0), mu);   // copy through exactly
            } else {
#pragma unroll
                for (int e = 0; e < LT::kVec; ++e) mu[e] = M[m * LT::kVec + e] / I[m * LT::kVec + e];
            }
#pragma unroll
            for (int e = 0; e < LT::kVec; ++e) ii[e] = I[m * LT::kVec + e];
            vecf<LT::kVec>::st(a.muT + srow + LT::col(g, m, 0), mu);
            vecf<LT::kVec>::st(a.IT + srow + LT::col(g, m, 0), ii);
        }
    }
}

// ---------------------------------------------------------------------------
// time-split summary pass on the matrix cores
// ---------------------------------------------------------------------------
//
// A segment's affine summary from a zero state is a sum of decayed outer
// products (the natural-parameter scans of slides frame "Natural parameters
// expose two affine scans", App. A.12, unrolled over the segment):
//
//     M_loc    = sum_s w_s (beta_s . v_s) (x) k_s,     w_s = prod_{r > s} alpha_r
//     Ibar_loc = sum_s w_s  beta_s         (x) k_s^2,   P   = prod_s alpha_s
//
// a dense contraction over the segment's tokens, so it runs on
// v_mfma_f32_16x16x4_f32 (float32 operands and accumulation) instead of the
// recurrence's 4 VALU ops per entry and token.  Per chunk of 64 staged tokens
// the accumulators are first scaled by the chunk's decay P_c and then take
// the chunk's 64 outer products weighted by w within the chunk,
// w_t = exp(sum_{r > t} -A dt_r) (a suffix sum over at most 63 tokens, so no
// long products).
//
// One workgroup per (segment, head, 16 value rows, 64 key columns); wave w
// owns the 16-column tiles w, w + 4, ... of its slice of M_loc and of Ibar_loc.  Operand
// layout of v_mfma_f32_16x16x4_f32 (A 16x4, B 4x16, C 16x16): lane l gives
// A[l % 16][l / 16] and B[l / 16][l % 16] and holds C[4 (l / 16) + r][l % 16],
// r = 0..3; here the 4-wide inner dimension is 4 tokens, A's rows are value
// rows and B's columns are key columns.
// DPP moves for a wave scan: lanes whose source is out of range read 0
// (dpp_zero), or only the rows in ROWS take part and the others add 0.
template <int CTRL>
__device__ inline float dpp_zero(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
template <int CTRL, int ROWS>
__device__ inline float dpp_rows(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xF, false));
}

// Staging of the summary pass: chunks of 64 tokens kept in LDS in the input
// type and in the input's layout (k as [token][column], v and beta as
// [token][row]), written with 16-byte stores, plus the chunk-local weights
// w_t and the chunk's decay.  The matrix-core operands need one column (or
// row) per lane and successive tokens per step, so bf16 inputs are read back
// with gfx950's transposing LDS read (ds_read_b64_tr_b16: four tokens of the
// lane's column per read) and float32 inputs one value at a time.  k rows are
// 80 elements apart (a 64-column slice plus padding), so that the 16 lanes of
// a transposing read (4 rows x 4 column quads) hit 32 distinct banks.  The
// global loads of chunk c+1 are in flight while chunk c is on the matrix
// cores.
template <int DK, typename TIn>
struct SumStage {
    static constexpr int C = 64;
    static constexpr int kPer = 16 / (int)sizeof(TIn);         // elements per 16-byte packet
    static constexpr int kRS = DK <= 64 ? 80 : DK + 16;         // k row stride (elements)
    static constexpr int kColPkts = DK / kPer;
    static constexpr int kRowPkts = kRowsPerWG / kPer;         // packets per token of v (or beta)
    static constexpr int kKP = C * kColPkts;
    static constexpr int kKPT = kKP / kThreads;
    static constexpr int kVP = C * kRowPkts;
    static constexpr int kVPT = (2 * kVP + kThreads - 1) / kThreads;
    static constexpr size_t kKBytes = (size_t)C * kRS * sizeof(TIn);
    static constexpr size_t kVBytes = (size_t)C * kRowsPerWG * sizeof(TIn);
    static constexpr size_t kBuf = kKBytes + 2 * kVBytes + (size_t)(C + 4) * sizeof(float);
    static_assert(kKP % kThreads == 0 && C <= kThreads, "whole packets per thread");

    uint4 kp[kKPT], vp[kVPT];
    uint32_t dtv = 0;

    // k rows are DK wide here but ktok elements apart in memory (a slice of a
    // wider head when the key columns are split over workgroups)
    __device__ inline void load(const TIn *kb, const TIn *vb, const TIn *bb, const TIn *db, int left, int H,
                                int dv, uint32_t ktok, int tid) {
#pragma unroll
        for (int u = 0; u < kKPT; ++u) {
            const int p = tid + u * kThreads;
            const int tt = p / kColPkts;
            kp[u] = make_uint4(0, 0, 0, 0);
            if (tt < left) kp[u] = *(const uint4 *)(kb + (uint32_t)tt * ktok + (p % kColPkts) * kPer);
        }
#pragma unroll
        for (int u = 0; u < kVPT; ++u) {
            const int q = tid + u * kThreads;
            if (q < 2 * kVP) {
                const bool isb = q >= kVP;
                const int pp = isb ? q - kVP : q;
                const int tt = pp / kRowPkts;
                vp[u] = make_uint4(0, 0, 0, 0);
                if (tt < left)
                    vp[u] = *(const uint4 *)((isb ? bb : vb) + (uint32_t)tt * (uint32_t)(H * dv) + (pp % kRowPkts) * kPer);
            }
        }
        if (tid < C) {
            dtv = 0;
            if (tid < left) dtv = io<TIn>::bits(db[(uint32_t)tid * (uint32_t)H]);
        }
    }

    // Packets to LDS; wave 0 forms the chunk's weights: with l_t = -A dt_t,
    // w_t = exp(sum_{r > t} l_r) (an exclusive suffix sum over the 64 lanes)
    // and the chunk's decay P_c = w_0 exp(l_0).
    __device__ inline void commit(char *buf, float A, int tid) const {
        TIn *kl = (TIn *)buf;
        TIn *vl = (TIn *)(buf + kKBytes);
        TIn *bl = (TIn *)(buf + kKBytes + kVBytes);
        float *gl = (float *)(buf + kKBytes + 2 * kVBytes);
#pragma unroll
        for (int u = 0; u < kKPT; ++u) {
            const int p = tid + u * kThreads;
            *(uint4 *)(kl + (p / kColPkts) * kRS + (p % kColPkts) * kPer) = kp[u];
        }
#pragma unroll
        for (int u = 0; u < kVPT; ++u) {
            const int q = tid + u * kThreads;
            if (q < 2 * kVP) {
                const bool isb = q >= kVP;
                const int pp = isb ? q - kVP : q;
                *(uint4 *)((isb ? bl : vl) + (pp / kRowPkts) * kRowsPerWG + (pp % kRowPkts) * kPer) = vp[u];
            }
        }
        if (tid < 64) {
            // token t sits in lane 63 - t, so a prefix scan over the lanes is a
            // suffix sum over the tokens; shifting by one lane first makes it
            // exclusive (a lane's own token is not in its sum)
            const float l = -A * io<TIn>::from_bits(dtv);
            const float x = __shfl(l, 63 - tid, 64);
            float e = dpp_zero<0x138>(x);                    // wave_shr:1
            e += dpp_zero<0x111>(e);                         // row_shr:1
            e += dpp_zero<0x112>(e);                         // row_shr:2
            e += dpp_zero<0x114>(e);                         // row_shr:4
            e += dpp_zero<0x118>(e);                         // row_shr:8
            e += dpp_rows<0x142, 0xA>(e);                    // row_bcast:15 into rows 1, 3
            e += dpp_rows<0x143, 0xC>(e);                    // row_bcast:31 into rows 2, 3
            const float et = __shfl(e, 63 - tid, 64);        // back to token order
            const float wt = expf(et);
            gl[tid] = wt;
            if (tid == 0) gl[C] = wt * expf(l);
        }
    }

    // Lane (g, m) = (lane / 16, lane % 16): X[r0 + 8 g + e][c0 + m], e = 0..3,
    // widened (rows of rs elements).
    __device__ static inline void read4(const TIn *X, int rs, int r0, int c0, int lane, float *o) {
        const int g = lane >> 4, m = lane & 15;
        if constexpr (sizeof(TIn) == 2) {
            typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
            const TIn *p = X + (r0 + 8 * g + (m >> 2)) * rs + c0 + 4 * (m & 3);
            const i16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = __uint_as_float((uint32_t)(uint16_t)x[e] << 16);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = io<TIn>::to_f32(X[(r0 + 8 * g + e) * rs + c0 + m]);
        }
    }
};

template <int DK, typename TIn>
__global__ __launch_bounds__(kThreads) void summary_mfma_kernel(FwdArgs a) {
    // each workgroup owns 16 value rows and a slice of DKC key columns
    constexpr int kCS = DK >= 64 ? DK / 64 : 1;
    constexpr int DKC = DK / kCS;
    using SS = SumStage<DKC, TIn>;
    constexpr int C = SS::C;
    constexpr int kTiles = DKC / 16;
    constexpr int kTPW = (kTiles + kWaves - 1) / kWaves;   // tiles per wave (at most)
    extern __shared__ float lds[];
    char *buf0 = (char *)lds;
    char *buf1 = buf0 + SS::kBuf;

    const int rb_per_head = a.dv / kRowsPerWG;
    int wg = blockIdx.x;
    if (a.xcd_remap) {
        const int per_xcd = a.nwg / 8;
        wg = (wg % 8) * per_xcd + wg / 8;
    }
    const int cs = wg % kCS;
    wg /= kCS;
    const int seg = wg / a.nwg_seg;
    wg -= seg * a.nwg_seg;
    const int bh = wg / rb_per_head;
    const int row0 = (wg % rb_per_head) * kRowsPerWG;
    const int col0 = cs * DKC;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar tile tests
    const SegWs w(a.ws, a.nseg, (size_t)a.B * a.H, a.dv, DK);

    if (seg == 0 && cs == 0 && a.mu0) {   // the replay pass's copy of the start state (see SegWs)
        const size_t base = ((size_t)bh * a.dv + row0) * DK;
        for (int n = 4 * tid; n < kRowsPerWG * DK; n += 4 * kThreads) {
            *(float4 *)(w.mu0 + base + n) = *(const float4 *)(a.mu0 + base + n);
            *(float4 *)(w.I0 + base + n) = *(const float4 *)(a.I0 + base + n);
        }
    }

    const int t_begin = seg * a.seg_len;
    const int ntok = min(a.T, t_begin + a.seg_len) - t_begin;
    const int nchunks = (ntok + C - 1) / C;
    const size_t seq = ((size_t)b * a.T + t_begin) * a.H + h;
    const TIn *kseq = (const TIn *)a.k + seq * DK + col0;
    const TIn *vseq = (const TIn *)a.v + seq * a.dv + row0;
    const TIn *bseq = (const TIn *)a.beta + seq * a.dv + row0;
    const TIn *dseq = (const TIn *)a.dt + seq;
    const size_t kq_tok = (size_t)a.H * DK, vb_tok = (size_t)a.H * a.dv;
    const float A = a.A[h];
    const bool vstar = a.vstar != 0;

    f32x4 accM[kTPW], accI[kTPW];
#pragma unroll
    for (int t = 0; t < kTPW; ++t) { accM[t] = f32x4{0.f, 0.f, 0.f, 0.f}; accI[t] = f32x4{0.f, 0.f, 0.f, 0.f}; }
    float P = 1.f;
    const int m = lane & 15, kq = lane >> 4;     // A row / B column; token within the 4-token step

    SS st;
    if (nchunks > 0) {
        st.load(kseq, vseq, bseq, dseq, ntok, a.H, a.dv, (uint32_t)kq_tok, tid);
        st.commit(buf0, A, tid);
        __syncthreads();
    }
    for (int c = 0; c < nchunks; ++c) {
        const bool more = c + 1 < nchunks;
        if (more) {
            const size_t tn = (size_t)((c + 1) * C);
            st.load(kseq + tn * kq_tok, vseq + tn * vb_tok, bseq + tn * vb_tok, dseq + tn * a.H,
                    ntok - (c + 1) * C, a.H, a.dv, (uint32_t)kq_tok, tid);
        }
        const char *cur = (c & 1) ? buf1 : buf0;
        const TIn *kl = (const TIn *)cur;
        const TIn *vl = (const TIn *)(cur + SS::kKBytes);
        const TIn *bl = (const TIn *)(cur + SS::kKBytes + SS::kVBytes);
        const float *gl = (const float *)(cur + SS::kKBytes + 2 * SS::kVBytes);
        // decay of the whole chunk applied to what came before it
        const float Pc = gl[C];
        P *= Pc;
#pragma unroll
        for (int t = 0; t < kTPW; ++t) { accM[t] *= Pc; accI[t] *= Pc; }
        // steps of 4 tokens: lane group g feeds token r0 + 8 g + e at step (r0, e),
        // r0 in {0, 4, 32, 36}, so the 16 steps cover the 64 tokens once
#pragma unroll
        for (int r0i = 0; r0i < 4; ++r0i) {
            const int r0 = (r0i >> 1) * 32 + (r0i & 1) * 4;
            const float4 w4 = *(const float4 *)(gl + r0 + 8 * kq);
            const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
            float v4[4], b4[4];
            SS::read4(vl, kRowsPerWG, r0, 0, lane, v4);
            SS::read4(bl, kRowsPerWG, r0, 0, lane, b4);
#pragma unroll
            for (int t = 0; t < kTPW; ++t) {
                const int tile = wave + kWaves * t;
                if (kTiles % kWaves == 0 || tile < kTiles) {
                    float k4[4];
                    SS::read4(kl, SS::kRS, r0, tile * 16, lane, k4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float aI = wv[e] * b4[e];
                        const float aM = vstar ? wv[e] * v4[e] : aI * v4[e];   // w beta v, or w v*
                        accM[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(aM, k4[e], accM[t], 0, 0, 0);
                        accI[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(aI, k4[e] * k4[e], accI[t], 0, 0, 0);
                    }
                }
            }
        }
        if (more) st.commit((c & 1) ? buf0 : buf1, A, tid);
        __syncthreads();
    }

    // lane l holds rows 4 (l / 16) + r, column l % 16 of each of its tiles
#pragma unroll
    for (int t = 0; t < kTPW; ++t) {
        const int tile = wave + kWaves * t;
        if (kTiles % kWaves == 0 || tile < kTiles) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const size_t o = ((size_t)bh * a.dv + row0 + 4 * kq + r) * DK + col0 + tile * 16 + m;
                w.M[seg * w.per_seg + o] = accM[t][r];
                w.Ib[seg * w.per_seg + o] = accI[t][r];
            }
        }
    }
    if (row0 == 0 && cs == 0 && tid == 0) w.P[(size_t)seg * a.B * a.H + bh] = P;
}

// ---------------------------------------------------------------------------
// backward (training): reverse mode of the chunked forward
// ---------------------------------------------------------------------------
//
// The pages train through the recurrence but print no backward; this is the
// adjoint of the natural-parameter scans (slides, frame "Natural parameters
// expose two affine scans", App. A.12) per state entry (i, j):
//     M_t = a_t M_{t-1} + bv_i k_j,   I_t = a_t I_{t-1} + c_t + b_i k_j^2,
//     y_t[i] = sum_j (M_t / I_t) q_j,   a = e^{-A dt},  c = (1 - a) I_prior.
// With GM, GI the adjoints of (M_t, I_t), r = 1 / I_t and mu = M_t r, walking
// t from T-1 down to 0:
//     GM += gy_i q_j r,         GI -= gy_i q_j r mu           (readout)
//     gq_j += gy_i mu,          gk_j += GM bv_i + 2 GI b_i k_j
//     gbv_i += GM k_j,          gb_i += GI k_j^2
//     da_t += GM M_{t-1} + GI I_{t-1},     dc_t += GI
//     GM *= a_t,  GI *= a_t                                    (to t-1)
// and then gv = gbv b, gbeta = gbv v + gb, gdt = A a (I_prior dc - da),
// gA = sum dt a (I_prior dc - da), gI_prior = sum (1 - a) dc.  The adjoint
// of the final state (mu_T = M_T / I_T, I_T) starts the walk:
// GM = gmuT / I_T, GI = gIT - GM mu_T; at the start M_0 = I_0 mu_0 gives
// gmu0 = GM I_0 and gI0 = GI + GM mu_0.
//
// Passes (one stream):
//  1. checkpoint: the forward kernel in kCheckpoint mode stores (M, I)
//     before every 16th token (4 VALU ops per entry and token, no readout).
//  2. bwd_kernel: one workgroup per (head, 16 value rows), the forward's
//     lane layout.  Sub-blocks of 8 tokens are taken newest first, each
//     16-token checkpoint interval as its newer sub-block, then its older one.
//     The newer one first replays the older one from the checkpoint to reach
//     its own start state, leaving the state at the older one's token 4 in a
//     per-thread LDS snapshot.  In each sub-block each half of 4 tokens is
//     replayed into registers (from the sub-block's start state, or from the
//     snapshot for the older sub-block's upper half) and walked in reverse:
//     28 replayed tokens per interval, against 24 with a checkpoint every 8
//     tokens, for half the checkpoint bytes.  Row sums (gbv, gb, da, dc) use the forward's transposing
//     DPP reduction; column sums (gq, gk) are reduce-scattered across the
//     4 rows of a wave, summed over the 4 waves in LDS and written as this
//     row block's partial.
//  3. bwd_qk_kernel sums the row-block partials into gq, gk;
//     bwd_gate_kernel forms gdt and per-sequence sums of the gate gradients;
//     bwd_head_kernel sums those over the batch into gA, gI_prior.

template <int DK> struct BwdStage {
    static constexpr int kColFloats = 3 * DK;                 // k, k^2, q
    static constexpr int kRowFloats = 4 * kRowsPerWG;         // (beta, beta v, v, gy) per row
    static constexpr int kRows = kSB * kColFloats;
    static constexpr int kGate = kRows + kSB * kRowFloats;    // (alpha, c) per token
    static constexpr int kFloats = kGate + 2 * kSB;
    static constexpr int kRed = 2 * kFloats;                  // gq | gk per token and wave
    static constexpr int kRs = kRed + kSB * kWaves * 2 * DK;   // row sums [token][4][16 rows]
    // per-thread snapshot of (M, I) at an older sub-block's token 4: float4 i
    // of thread tid at kSnap + 4 (i kThreads + tid)
    static constexpr int kSnap = kRs + kSB * 4 * kRowsPerWG;
    static constexpr int kTotal = kSnap + kThreads * 2 * (DK / kLanesPerRow);
};

struct BwdArgs {
    const void *q, *k, *v, *beta, *dt, *gy;
    const float *A, *Ip, *mu0, *I0, *gmuT, *gIT;
    float *gv, *gbeta, *gmu0, *gI0;
    const float *ck;
    float *pqk;        // [row block][B*T*H][2 DK]: gq | gk partials
    float *ps;         // [row block][B*H][T][2]: (da, dc) partials
    float *pI0;        // [B*H][row block]: sum of gI0 (default start state)
    float *pip;        // per-entry prior: [B*H][dv][dk] per-sequence gradient of I_prior
    int B, T, H, dv, nwg, xcd_remap;
    int nsb;           // sub-blocks per sequence: ceil(T / kSB)
    int nck;           // checkpoints per sequence: ceil(T / kCkI)
    int vstar;         // 1: v holds beta . v
};

// Staging of one sub-block of kSB tokens (newest-first order of use; the
// layout is that of the forward with q always present and per-row gy, v).
template <int DK, typename TIn, typename TG>
struct BwdStager {
    static constexpr int kPer = packet<TIn>::kN;
    static constexpr int kColPkts = DK / kPer;
    static constexpr int kHalf = kSB * kColPkts;              // k packets (= q packets)
    static constexpr int kKQPer = (2 * kHalf + kThreads - 1) / kThreads;
    static constexpr int kRowPkts = kRowsPerWG / kPer;
    static constexpr int kVB = kSB * kRowPkts;
    static constexpr int kPerG = packet<TG>::kN;
    static constexpr int kRowPktsG = kRowsPerWG / kPerG;
    static constexpr int kGY = kSB * kRowPktsG;
    static_assert(kVB <= kThreads && kGY <= kThreads, "one packet per thread");

    uint4 kq[kKQPer];
    uint4 vv, bb, gg;
    uint32_t dtv;          // raw bits (io<TIn>::bits) until the commit
    int left_;             // tokens of the sequence from the sub-block's start

    // Makes the loaded packets count as used here, so the wait for them lands
    // here rather than at the commit, after the walk's stores.
    __device__ inline void ready() const {
#pragma unroll
        for (int u = 0; u < kKQPer; ++u) asm volatile("" ::"v"(kq[u].x), "v"(kq[u].y), "v"(kq[u].z), "v"(kq[u].w));
        asm volatile("" ::"v"(vv.x), "v"(vv.y), "v"(vv.z), "v"(vv.w), "v"(bb.x), "v"(bb.y), "v"(bb.z), "v"(bb.w));
        asm volatile("" ::"v"(gg.x), "v"(gg.y), "v"(gg.z), "v"(gg.w), "v"(dtv));
    }

    __device__ static inline int vb_slot(int tid) { return (tid + kThreads - 64) % kThreads; }
    __device__ static inline int gy_slot(int tid) { return (tid + kThreads - 128) % kThreads; }
    __device__ static inline int dt_slot(int tid) { return (tid + kThreads - 192) % kThreads; }

    // Bases point at token t0 of this (b, h) (v, beta, gy at the workgroup's
    // first row); `left` = T - t0 >= 1.  Token tt is at offset tt H d.
    // Branch-free: every thread issues every load, tokens past the end read
    // token left - 1 (the commit stages zeros for them) and threads without a
    // packet read packet 0.  Loads under per-lane branches are not counted by
    // the compiler, which then makes the next wait for an earlier load (a
    // checkpoint) wait for all of these as well.
    __device__ inline void load(const TIn *kb, const TIn *qb, const TIn *vb, const TIn *bb_, const TG *gb,
                                const TIn *db, int left, int H, int dv, int tid) {
        left_ = left;
#pragma unroll
        for (int u = 0; u < kKQPer; ++u) {
            int p = tid + u * kThreads;
            if ((2 * kHalf) % kThreads != 0 && p >= 2 * kHalf) p = 0;
            const bool isq = p >= kHalf;
            const int pp = isq ? p - kHalf : p;
            const int tt = min(pp / kColPkts, left - 1);
            const uint32_t off = (uint32_t)tt * (uint32_t)(H * DK) + (pp % kColPkts) * kPer;
            kq[u] = *(const uint4 *)((isq ? qb : kb) + off);
        }
        {
            const int pv = vb_slot(tid) < kVB ? vb_slot(tid) : 0;
            const int tt = min(pv / kRowPkts, left - 1);
            const uint32_t off = (uint32_t)tt * (uint32_t)(H * dv) + (pv % kRowPkts) * kPer;
            vv = *(const uint4 *)(vb + off);
            bb = *(const uint4 *)(bb_ + off);
        }
        {
            const int pg = gy_slot(tid) < kGY ? gy_slot(tid) : 0;
            const int tt = min(pg / kRowPktsG, left - 1);
            const uint32_t off = (uint32_t)tt * (uint32_t)(H * dv) + (pg % kRowPktsG) * kPerG;
            gg = *(const uint4 *)(gb + off);
        }
        {
            const int pd = dt_slot(tid) < kSB ? dt_slot(tid) : 0;
            dtv = io<TIn>::bits(db[(uint32_t)min(pd, left - 1) * (uint32_t)H]);
        }
    }

    __device__ inline void commit(float *buf, float A, float Ip, int tid, bool vstar) const {
        using S = BwdStage<DK>;
        float *rows = buf + S::kRows;
#pragma unroll
        for (int u = 0; u < kKQPer; ++u) {
            const int p = tid + u * kThreads;
            if ((2 * kHalf) % kThreads == 0 || p < 2 * kHalf) {
                const bool isq = p >= kHalf;
                const int pp = isq ? p - kHalf : p;
                const int tt = pp / kColPkts;
                const int off = (pp % kColPkts) * kPer;
                float x[kPer];
                packet<TIn>::widen(tt < left_ ? kq[u] : make_uint4(0, 0, 0, 0), x);   // past the end: k = q = 0
                float *dst = buf + tt * S::kColFloats + off;
#pragma unroll
                for (int e = 0; e < kPer; e += 4) {
                    if (!isq) {
                        *(float4 *)(dst + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
                        *(float4 *)(dst + DK + e) = make_float4(x[e] * x[e], x[e + 1] * x[e + 1],
                                                                x[e + 2] * x[e + 2], x[e + 3] * x[e + 3]);
                    } else {
                        *(float4 *)(dst + 2 * DK + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
                    }
                }
            }
        }
        const int pv = vb_slot(tid);
        if (pv < kVB) {
            const int tt = pv / kRowPkts;
            const int r0 = (pv % kRowPkts) * kPer;
            const bool in = tt < left_;       // past the end: v = beta = 0
            float xv[kPer], xb[kPer];
            packet<TIn>::widen(in ? vv : make_uint4(0, 0, 0, 0), xv);
            packet<TIn>::widen(in ? bb : make_uint4(0, 0, 0, 0), xb);
            float *dst = rows + tt * S::kRowFloats + 4 * r0;
#pragma unroll
            for (int e = 0; e < kPer; ++e) {
                *(float2 *)(dst + 4 * e) = make_float2(xb[e], vstar ? xv[e] : xb[e] * xv[e]);
                dst[4 * e + 2] = xv[e];
            }
        }
        const int pg = gy_slot(tid);
        if (pg < kGY) {
            const int tt = pg / kRowPktsG;
            const int r0 = (pg % kRowPktsG) * kPerG;
            float xg[kPerG];
            packet<TG>::widen(tt < left_ ? gg : make_uint4(0, 0, 0, 0), xg);
            float *dst = rows + tt * S::kRowFloats + 4 * r0 + 3;
#pragma unroll
            for (int e = 0; e < kPerG; ++e) dst[4 * e] = xg[e];
        }
        const int pd = dt_slot(tid);
        if (pd < kSB) {
            // past the end: dt = 0, so alpha = 1 and c = 0
            const float2 gc = gate(A, io<TIn>::from_bits(pd < left_ ? dtv : 0u), Ip);
            *(float2 *)(buf + S::kGate + 2 * pd) = gc;
        }
    }
};

// One token of the replay: the forward update of the lane's entries (the
// same operations as compute_chunk, so the states are bit-identical).  FZ
// (frozen importance) replays the content scan only.
template <int DK, bool IPE, bool FZ = false>
__device__ inline void bwd_replay_token(const float *buf, int e, float *M, float *I, int row_local, int g,
                                        const float *ipe) {
    using LT = LaneTile<DK>;
    using S = BwdStage<DK>;
    const float2 gc = *(const float2 *)(buf + S::kGate + 2 * e);
    const float2 rb = *(const float2 *)(buf + S::kRows + e * S::kRowFloats + 4 * row_local);
    const float *ct = buf + e * S::kColFloats + LT::col(g, 0, 0);
#pragma unroll
    for (int m = 0; m < LT::kNVec; ++m) {
        float kk[LT::kVec], k2[LT::kVec];
        const int c0 = kLanesPerRow * LT::kVec * m;
        vecf<LT::kVec>::ld(ct + c0, kk);
        vecf<LT::kVec>::ld(ct + DK + c0, k2);
#pragma unroll
        for (int x = 0; x < LT::kVec; ++x) {
            const int s = m * LT::kVec + x;
            if (!FZ) {
                const float w = fmaf(rb.x, k2[x], IPE ? gc.y * ipe[s] : gc.y);
                I[s] = fmaf(gc.x, I[s], w);
            }
            M[s] = fmaf(gc.x, M[s], rb.y * kk[x]);
        }
    }
}

// Reduce-scatter of a token's (gq, gk) lane partials over the wave's 4 rows.
// v_permlane32_swap of (x, y) leaves lanes < 32 with x of lanes l and l+32
// and the others with y of lanes l-32 and l, so one add pairs rows (0, 2) and
// (1, 3) and keeps gq in the low half-wave, gk in the high; v_permlane16_swap
// then pairs rows (0, 1) and (2, 3), even rows keeping the first half of the
// lane's columns.  The wave's column sums land in red (2 DK floats).
template <int DK>
__device__ inline void bwd_scatter_qk(const float *dq, const float *dk, int lane, int g, float *red) {
    using LT = LaneTile<DK>;
    constexpr int KC = LT::kCols;
    const bool up32 = lane & 32, up16 = lane & 16;
    float h8[KC];
#pragma unroll
    for (int s = 0; s < KC; ++s) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(dq[s]), __float_as_uint(dk[s]), false, false);
        h8[s] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    constexpr int KH = KC / 2;
    float h4[KH];
#pragma unroll
    for (int s = 0; s < KH; ++s) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(h8[s]), __float_as_uint(h8[KH + s]), false, false);
        h4[s] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const int s0 = up16 ? KH : 0;
    float *dst = red + (up32 ? DK : 0) + LT::col(g, s0 / LT::kVec, s0 % LT::kVec);
    if (KH == 4) *(float4 *)dst = make_float4(h4[0], h4[KH > 1 ? 1 : 0], h4[KH > 2 ? 2 : 0], h4[KH > 3 ? 3 : 0]);
    else if (KH == 2) *(float2 *)dst = make_float2(h4[0], h4[KH > 1 ? 1 : 0]);
    else dst[0] = h4[0];
}

// One token of the reverse walk for the lane's entries: (Mt, It) the state
// after the token, (Mp, Ipv) before it.  Updates the adjoints, returns the
// lane's row partials of (gbv, gb, da, dc), and writes the wave's column sums
// of (gq, gk) for the token to red (2 DK floats), reduce-scattered over the
// wave's 4 rows: after exchanges with lanes l^32 and l^16, lane (rg, g) holds
// DK/32 consecutive columns of gq (rg < 2) or gk (rg >= 2).  With a prior per
// entry (IPE) dc is sum Ip_ij GI_ij (the staged c is 1 - alpha) and accIp
// collects the entry's own gradient, sum_t (1 - alpha_t) GI_ij.
template <int DK, bool IPE>
__device__ inline void bwd_reverse_token(const float *buf, int e, const float *Mt, const float *It,
                                         const float *Mp, const float *Ipv, float *GM, float *GI,
                                         int row_local, int g, int lane, float *red,
                                         float &cbv, float &cb, float &s1, float &s2,
                                         const float *ipe, float *accIp) {
    using LT = LaneTile<DK>;
    using S = BwdStage<DK>;
    constexpr int KC = LT::kCols;
    const float2 gate_e = *(const float2 *)(buf + S::kGate + 2 * e);
    const float alpha = gate_e.x;
    const float4 rw = *(const float4 *)(buf + S::kRows + e * S::kRowFloats + 4 * row_local);
    const float b2 = 2.f * rw.x, bv = rw.y, gy = rw.w;
    const float *ct = buf + e * S::kColFloats + LT::col(g, 0, 0);
    float dq[KC], dk[KC];
    cbv = 0.f; cb = 0.f; s1 = 0.f; s2 = 0.f;
#pragma unroll
    for (int m = 0; m < LT::kNVec; ++m) {
        float kk[LT::kVec], k2[LT::kVec], qq[LT::kVec];
        const int c0 = kLanesPerRow * LT::kVec * m;
        vecf<LT::kVec>::ld(ct + c0, kk);
        vecf<LT::kVec>::ld(ct + DK + c0, k2);
        vecf<LT::kVec>::ld(ct + 2 * DK + c0, qq);
#pragma unroll
        for (int x = 0; x < LT::kVec; ++x) {
            const int s = m * LT::kVec + x;
            // readout adjoint: with u = q r, GM += gy u and GI -= gy q r mu = dq u
            const float r = __builtin_amdgcn_rcpf(It[s]);
            const float u = qq[x] * r;
            const float mu = Mt[s] * r;
            GM[s] = fmaf(gy, u, GM[s]);
            dq[s] = gy * mu;
            GI[s] = fmaf(-dq[s], u, GI[s]);
            dk[s] = fmaf(GM[s], bv, GI[s] * (b2 * kk[x]));
            cbv = fmaf(GM[s], kk[x], cbv);
            cb = fmaf(GI[s], k2[x], cb);
            s1 = fmaf(GM[s], Mp[s], s1);
            s1 = fmaf(GI[s], Ipv[s], s1);
            if (IPE) {
                s2 = fmaf(ipe[s], GI[s], s2);
                accIp[s] = fmaf(gate_e.y, GI[s], accIp[s]);
            } else {
                s2 += GI[s];
            }
            GM[s] *= alpha;
            GI[s] *= alpha;
        }
    }
    bwd_scatter_qk<DK>(dq, dk, lane, g, red);
}

// One token of the frozen-importance reverse walk (the importance held at
// I_prior, the Mamba2 limit): the content scan M_t = a_t M_{t-1} + bv_i k_j is
// the exact path's, the readout is y_t = M_t q_t / I_prior.  With GM the
// adjoint of M_t: GM += gy_i q_j / I_prior, gq_j += gy_i M_ij / I_prior,
// gk_j += GM bv_i, gbv_i += GM k_j, da_t += GM M_{t-1}, GM *= a_t.
template <int DK>
__device__ inline void bwd_reverse_token_fz(const float *buf, int e, const float *Mt, const float *Mp, float *GM,
                                            int row_local, int g, int lane, float *red, float &cbv, float &s1,
                                            float rIp) {
    using LT = LaneTile<DK>;
    using S = BwdStage<DK>;
    constexpr int KC = LT::kCols;
    const float alpha = buf[S::kGate + 2 * e];
    const float4 rw = *(const float4 *)(buf + S::kRows + e * S::kRowFloats + 4 * row_local);
    const float bv = rw.y, gyr = rw.w * rIp;
    const float *ct = buf + e * S::kColFloats + LT::col(g, 0, 0);
    float dq[KC], dk[KC];
    cbv = 0.f; s1 = 0.f;
#pragma unroll
    for (int m = 0; m < LT::kNVec; ++m) {
        float kk[LT::kVec], qq[LT::kVec];
        const int c0 = kLanesPerRow * LT::kVec * m;
        vecf<LT::kVec>::ld(ct + c0, kk);
        vecf<LT::kVec>::ld(ct + 2 * DK + c0, qq);
#pragma unroll
        for (int x = 0; x < LT::kVec; ++x) {
            const int s = m * LT::kVec + x;
            GM[s] = fmaf(gyr, qq[x], GM[s]);
            dq[s] = gyr * Mt[s];
            dk[s] = GM[s] * bv;
            cbv = fmaf(GM[s], kk[x], cbv);
            s1 = fmaf(GM[s], Mp[s], s1);
            GM[s] *= alpha;
        }
    }
    bwd_scatter_qk<DK>(dq, dk, lane, g, red);
}

// Row sums of one half-block: acc holds the lane's partials of (gbv, gb, da,
// dc) for 4 tokens, quantity-major.  After the transposing reduction lane g
// holds quantity g / 4 of token g % 4 summed over its row; it is written to
// dst[(token * 4 + quantity) * 16] (dst at this half's first token and the
// lane's row).
__device__ inline void bwd_row_sums(const float (&acc)[16], int g, float *dst) {
    const float r = row16_transpose_sum(acc, g);
    dst[((g % 4) * 4 + g / 4) * kRowsPerWG] = r;
}

// FZ: the backward of the frozen-importance forward (the importance held at
// I_prior): the same content scan, checkpoints and sums, with the importance
// terms dropped (see bwd_reverse_token_fz).
template <int DK, typename TIn, typename TG, bool IPE, bool FZ = false>
// Two workgroups per CU (its LDS allows two): with a prior per entry at d = 128
// this makes the compiler spill a few values rather than drop to one wave per
// SIMD, 9.8 ms instead of 11.6 ms on the 760M layer.
__global__ __launch_bounds__(kThreads, 2) void bwd_kernel(BwdArgs a) {
    using LT = LaneTile<DK>;
    using S = BwdStage<DK>;
    constexpr int KC = LT::kCols;
    extern __shared__ float lds[];
    float *red = lds + S::kRed;
    float *rs = lds + S::kRs;

    const int rb_per_head = a.dv / kRowsPerWG;
    int wg = blockIdx.x;
    if (a.xcd_remap) {
        const int per_xcd = a.nwg / 8;
        wg = (wg % 8) * per_xcd + wg / 8;
    }
    const int bh = wg / rb_per_head;
    const int rb = wg % rb_per_head;
    const int row0 = rb * kRowsPerWG;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane & (kLanesPerRow - 1);
    const int rg = lane >> 4;
    const int row_local = wave * kRowsPerWave + rg;
    const int row = row0 + row_local;
    const float A = a.A[h], Ip = IPE ? 1.f : a.Ip[h];
    const size_t srow = ((size_t)bh * a.dv + row) * DK;
    float ipe[IPE ? KC : 1], accIp[IPE ? KC : 1];
    if (IPE) {
        const float *ip = a.Ip + ((size_t)h * a.dv + row) * DK;
#pragma unroll
        for (int m = 0; m < LT::kNVec; ++m) vecf<LT::kVec>::ld(ip + LT::col(g, m, 0), ipe + m * LT::kVec);
#pragma unroll
        for (int s = 0; s < KC; ++s) accIp[s] = 0.f;
    }

    float GM[KC], GI[KC];
    if (FZ) {
#pragma unroll
        for (int s = 0; s < KC; ++s) GI[s] = 0.f;
    }
    const float rIp = 1.f / Ip;    // frozen importance: the readout divides by I_prior
    const size_t seq0 = (size_t)b * a.T * a.H + h;           // row of (b, 0, h) in [B, T, H]
    const size_t bth = (size_t)a.B * a.T * a.H;
    const size_t kq_tok = (size_t)a.H * DK, vb_tok = (size_t)a.H * a.dv;

    if (a.nsb == 0) {
        // T = 0: the final state is the initial state, copied through exactly
#pragma unroll
        for (int m = 0; m < LT::kNVec; ++m)
#pragma unroll
            for (int x = 0; x < LT::kVec; ++x) {
                const int s = m * LT::kVec + x;
                const size_t o = srow + LT::col(g, m, x);
                const float gmu = a.gmuT ? a.gmuT[o] : 0.f, gI = a.gIT ? a.gIT[o] : 0.f;
                if (a.gmu0) a.gmu0[o] = gmu;
                if (a.gI0) a.gI0[o] = gI;
                GI[s] = FZ ? 0.f : gI;
            }
    } else {
        const size_t ck_stride = (size_t)rb_per_head * kThreads * 2 * KC;
        const float *ckb = a.ck + ((size_t)bh * a.nck * rb_per_head + rb) * (kThreads * 2 * KC);
        const TIn *kseq = (const TIn *)a.k + seq0 * DK;
        const TIn *qseq = (const TIn *)a.q + seq0 * DK;
        const TIn *vseq = (const TIn *)a.v + seq0 * a.dv + row0;
        const TIn *bseq = (const TIn *)a.beta + seq0 * a.dv + row0;
        const TG *gseq = (const TG *)a.gy + seq0 * a.dv + row0;
        const TIn *dseq = (const TIn *)a.dt + seq0;
        float *snap = lds + S::kSnap;
        // Sub-block sb is staged in buffer sb & 1.  When sub-block sb starts,
        // sb and sb - 1 are both staged (a newer sub-block replays the older
        // one); sb - 2 is loaded during sb and committed into sb's buffer
        // after it.
        BwdStager<DK, TIn, TG> st;
        auto stage = [&](int sbl) __attribute__((always_inline)) {
            const size_t tn = (size_t)sbl * kSB;
            st.load(kseq + tn * kq_tok, qseq + tn * kq_tok, vseq + tn * vb_tok, bseq + tn * vb_tok,
                    gseq + tn * vb_tok, dseq + tn * a.H, a.T - (int)tn, a.H, a.dv, tid);
        };
        stage(a.nsb - 1);
        st.commit(lds + ((a.nsb - 1) & 1) * S::kFloats, A, Ip, tid, a.vstar);
        if (a.nsb > 1) {
            stage(a.nsb - 2);
            st.commit(lds + ((a.nsb - 2) & 1) * S::kFloats, A, Ip, tid, a.vstar);
        }
        // the start state of the current checkpoint interval (sub-blocks 2n, 2n + 1)
        float ckM[KC], ckI[KC];
        load_pair<KC>(ckb + (size_t)((a.nsb - 1) / 2) * ck_stride, tid, ckM, ckI);
        regs_ready<KC>(ckM);
        regs_ready<KC>(ckI);
        __syncthreads();

        for (int sb = a.nsb - 1; sb >= 0; --sb) {
            const float *cur = lds + (sb & 1) * S::kFloats;
            const int t0 = sb * kSB;
            const bool newer = sb & 1;      // the newer sub-block of its checkpoint interval
            if (sb > 1) stage(sb - 2);
            float nM[KC], nI[KC];           // the start state of the next sub-block taken
            if (newer) {
                // this sub-block's start state: the older sub-block (staged in
                // the other buffer) replayed from the interval's checkpoint,
                // which the older sub-block then starts from
                const float *older = lds + ((sb - 1) & 1) * S::kFloats;
#pragma unroll
                for (int s = 0; s < KC; ++s) { nM[s] = ckM[s]; nI[s] = ckI[s]; }
#pragma unroll
                for (int e = 0; e < 4; ++e) bwd_replay_token<DK, IPE, FZ>(older, e, ckM, ckI, row_local, g, ipe);
                lds_store_pair<KC>(snap, tid, ckM, ckI);
#pragma unroll
                for (int e = 4; e < 8; ++e) bwd_replay_token<DK, IPE, FZ>(older, e, ckM, ckI, row_local, g, ipe);
            }
            float xM[4][KC], xI[4][KC];
            float acc[16];      // this half's row partials: gbv, gb, da, dc of its 4 tokens
            // upper half: tokens 4..7, replayed from the state before token 4:
            // an older sub-block's snapshot, else the start state replayed
            float mM[KC], mI[KC];
            if (!newer && sb + 1 < a.nsb) {
                lds_load_pair<KC>(snap, tid, mM, mI);
            } else {
#pragma unroll
                for (int s = 0; s < KC; ++s) { mM[s] = ckM[s]; mI[s] = ckI[s]; }
#pragma unroll
                for (int e = 0; e < 4; ++e) bwd_replay_token<DK, IPE, FZ>(cur, e, mM, mI, row_local, g, ipe);
            }
#pragma unroll
            for (int e = 4; e < 8; ++e) {
                const float *pm = e == 4 ? mM : xM[e > 4 ? e - 5 : 0];
                const float *pi = e == 4 ? mI : xI[e > 4 ? e - 5 : 0];
#pragma unroll
                for (int s = 0; s < KC; ++s) { xM[e - 4][s] = pm[s]; xI[e - 4][s] = pi[s]; }
                bwd_replay_token<DK, IPE, FZ>(cur, e, xM[e - 4], xI[e - 4], row_local, g, ipe);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (sb == a.nsb - 1) {
                // adjoint of the final state (tokens past T are neutral: xM[3] is the state after T-1)
#pragma unroll
                for (int m = 0; m < LT::kNVec; ++m)
#pragma unroll
                    for (int x = 0; x < LT::kVec; ++x) {
                        const int s = m * LT::kVec + x;
                        const size_t o = srow + LT::col(g, m, x);
                        const float gmu = a.gmuT ? a.gmuT[o] : 0.f, gI = a.gIT ? a.gIT[o] : 0.f;
                        if (FZ) {
                            GM[s] = gmu * rIp;                  // mu_T = M_T / I_prior
                        } else {
                            const float muT = xM[3][s] / xI[3][s];
                            GM[s] = gmu / xI[3][s];
                            GI[s] = gI - GM[s] * muT;
                        }
                    }
            }
#pragma unroll
            for (int e = 7; e >= 4; --e) {
                if (FZ) {
                    bwd_reverse_token_fz<DK>(cur, e, xM[e - 4], e == 4 ? mM : xM[e > 4 ? e - 5 : 0], GM, row_local, g,
                                             lane, red + (e * kWaves + wave) * 2 * DK, acc[e - 4], acc[e + 4], rIp);
                    acc[e] = 0.f;
                    acc[e + 8] = 0.f;
                } else {
                    bwd_reverse_token<DK, IPE>(cur, e, xM[e - 4], xI[e - 4], e == 4 ? mM : xM[e > 4 ? e - 5 : 0],
                                               e == 4 ? mI : xI[e > 4 ? e - 5 : 0],
                                               GM, GI, row_local, g, lane, red + (e * kWaves + wave) * 2 * DK,
                                               acc[e - 4], acc[e], acc[e + 4], acc[e + 8], ipe, accIp);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            bwd_row_sums(acc, g, rs + 4 * 4 * kRowsPerWG + row_local);
            // lower half: tokens 0..3
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float *pm = e == 0 ? ckM : xM[e > 0 ? e - 1 : 0];
                const float *pi = e == 0 ? ckI : xI[e > 0 ? e - 1 : 0];
#pragma unroll
                for (int s = 0; s < KC; ++s) { xM[e][s] = pm[s]; xI[e][s] = pi[s]; }
                bwd_replay_token<DK, IPE, FZ>(cur, e, xM[e], xI[e], row_local, g, ipe);
                __builtin_amdgcn_sched_barrier(0);
            }
            // an older sub-block hands over to the previous interval's newer one
            if (!newer && sb > 0) load_pair<KC>(ckb + (size_t)(sb / 2 - 1) * ck_stride, tid, nM, nI);
#pragma unroll
            for (int e = 3; e >= 0; --e) {
                if (FZ) {
                    bwd_reverse_token_fz<DK>(cur, e, xM[e], e == 0 ? ckM : xM[e > 0 ? e - 1 : 0], GM, row_local, g,
                                             lane, red + (e * kWaves + wave) * 2 * DK, acc[e], acc[e + 8], rIp);
                    acc[e + 4] = 0.f;
                    acc[e + 12] = 0.f;
                } else {
                    bwd_reverse_token<DK, IPE>(cur, e, xM[e], xI[e], e == 0 ? ckM : xM[e > 0 ? e - 1 : 0],
                                               e == 0 ? ckI : xI[e > 0 ? e - 1 : 0],
                                               GM, GI, row_local, g, lane, red + (e * kWaves + wave) * 2 * DK,
                                               acc[e], acc[e + 4], acc[e + 8], acc[e + 12], ipe, accIp);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            bwd_row_sums(acc, g, rs + row_local);
            // the next sub-block's packets and start state, waited for while
            // only loads are outstanding (not after this sub-block's stores)
            if (sb > 1) st.ready();
            regs_ready<KC>(nM);
            regs_ready<KC>(nI);
            __syncthreads();
            // sums over the 4 waves: this row block's partials of (gq, gk) and (da, dc)
            for (int n = 4 * tid; n < kSB * 2 * DK; n += 4 * kThreads) {
                const int e = n / (2 * DK), c = n % (2 * DK);
                const float *r0 = red + e * kWaves * 2 * DK + c;
                const float4 v0 = *(const float4 *)r0, v1 = *(const float4 *)(r0 + 2 * DK);
                const float4 v2 = *(const float4 *)(r0 + 4 * DK), v3 = *(const float4 *)(r0 + 6 * DK);
                if (t0 + e < a.T)
                    *(float4 *)(a.pqk + ((size_t)rb * bth + seq0 + (size_t)(t0 + e) * a.H) * 2 * DK + c) =
                        make_float4((v0.x + v1.x) + (v2.x + v3.x), (v0.y + v1.y) + (v2.y + v3.y),
                                    (v0.z + v1.z) + (v2.z + v3.z), (v0.w + v1.w) + (v2.w + v3.w));
            }
            // per (token, row): gv = gbv beta, gbeta = gbv v + gb; per token: the
            // row block's sums of (da, dc)
            if (tid < kSB * kRowsPerWG) {
                const int e = tid / kRowsPerWG, r = tid % kRowsPerWG;
                const float gbv = rs[(e * 4 + 0) * kRowsPerWG + r], gb = rs[(e * 4 + 1) * kRowsPerWG + r];
                const float4 rw = *(const float4 *)(cur + S::kRows + e * S::kRowFloats + 4 * r);
                if (t0 + e < a.T) {
                    // the write is (beta v) k, or v* k: gv is then dL/dv* and beta
                    // enters only through the importance
                    const size_t o = (seq0 + (size_t)(t0 + e) * a.H) * a.dv + row0 + r;
                    a.gv[o] = a.vstar ? gbv : gbv * rw.x;
                    if (!FZ || a.gbeta) a.gbeta[o] = a.vstar ? gb : fmaf(gbv, rw.z, gb);
                }
            } else if (tid < kSB * kRowsPerWG + 2 * kSB) {
                const int u = tid - kSB * kRowsPerWG, e = u % kSB, qd = u / kSB;
                const float *src = rs + (e * 4 + 2 + qd) * kRowsPerWG;
                float v = 0.f;
                if (FZ && qd == 1) {
                    // frozen importance: sum_i gbv_i (beta v)_i, the prior's gradient
                    // through the readout's 1 / I_prior
#pragma unroll
                    for (int r = 0; r < kRowsPerWG; ++r)
                        v = fmaf(rs[e * 4 * kRowsPerWG + r],
                                 (cur + S::kRows + e * S::kRowFloats + 4 * r)[1], v);
                } else {
#pragma unroll
                    for (int r = 0; r < kRowsPerWG; ++r) v += src[r];
                }
                if (t0 + e < a.T) a.ps[((size_t)rb * bth + (size_t)bh * a.T + t0 + e) * 2 + qd] = v;
            }
            __syncthreads();
            if (sb > 1) {
                st.commit(lds + (sb & 1) * S::kFloats, A, Ip, tid, a.vstar);
                if (!newer) __syncthreads();    // sub-block sb - 1 replays sb - 2 at once
            }
            if (sb > 0) {
#pragma unroll
                for (int s = 0; s < KC; ++s) { ckM[s] = nM[s]; ckI[s] = nI[s]; }
            }
        }
        // gradients of the start state: M_0 = I_0 mu_0
#pragma unroll
        for (int m = 0; m < LT::kNVec; ++m)
#pragma unroll
            for (int x = 0; x < LT::kVec; ++x) {
                const int s = m * LT::kVec + x;
                const size_t o = srow + LT::col(g, m, x);
                if (FZ) {
                    if (a.gmu0) a.gmu0[o] = GM[s] * Ip;       // M_0 = I_prior mu_0
                    continue;
                }
                const float i0 = a.mu0 ? a.I0[o] : (IPE ? ipe[s] : Ip), m0 = a.mu0 ? a.mu0[o] : 0.f;
                const float gI0 = fmaf(GM[s], m0, GI[s]);
                if (a.gmu0) a.gmu0[o] = GM[s] * i0;
                if (a.gI0) a.gI0[o] = gI0;
                GI[s] = gI0;
            }
    }
    if (IPE) {
        // this sequence's gradient of the per-entry prior (the default start
        // state I0 = I_prior adds gI0 entry by entry)
#pragma unroll
        for (int m = 0; m < LT::kNVec; ++m)
#pragma unroll
            for (int x = 0; x < LT::kVec; ++x) {
                const int s = m * LT::kVec + x;
                a.pip[srow + LT::col(g, m, x)] = a.mu0 ? accIp[s] : accIp[s] + GI[s];
            }
    }
    // this row block's sum of gI0 (the default start state I0 = I_prior feeds gI_prior)
    float gs = 0.f;
#pragma unroll
    for (int s = 0; s < KC; ++s) gs += GI[s];
    gs = row16_sum(gs);
    gs += __shfl_xor(gs, 16, 64);
    gs += __shfl_xor(gs, 32, 64);
    __syncthreads();
    if (lane == 0) rs[wave] = gs;
    __syncthreads();
    if (tid == 0) a.pI0[(size_t)bh * rb_per_head + rb] = (rs[0] + rs[1]) + (rs[2] + rs[3]);
}

// gq, gk: sums of the row-block partials (4 floats per thread).
template <int DK>
__global__ __launch_bounds__(256) void bwd_qk_kernel(const float *pqk, float *gq, float *gk, size_t bth, int nrb) {
    const size_t n4 = (size_t)blockIdx.x * 256 + threadIdx.x;          // float4 index
    if (n4 >= bth * (2 * DK / 4)) return;
    // the row blocks' partials in order, 8 loads in flight at a time (a
    // rolled loop waited for each load before issuing the next); blocks
    // past nrb reload the last one and are not added
    constexpr int kU = 8;
    const size_t rs = bth * 2 * DK;
    float4 acc = *(const float4 *)(pqk + 4 * n4);
    for (int r0 = 1; r0 < nrb; r0 += kU) {
        float4 x[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int r = r0 + u < nrb ? r0 + u : nrb - 1;
            x[u] = *(const float4 *)(pqk + (size_t)r * rs + 4 * n4);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (r0 + u < nrb) { acc.x += x[u].x; acc.y += x[u].y; acc.z += x[u].z; acc.w += x[u].w; }
    }
    const size_t tok = (4 * n4) / (2 * DK);
    const int c = (int)((4 * n4) % (2 * DK));
    float *dst = c < DK ? gq + tok * DK + c : gk + tok * DK + (c - DK);
    *(float4 *)dst = acc;
}

// gdt per token and per-sequence sums of the gate gradients: one block per
// (b, h), tokens strided over its threads.
// (with a prior per entry dc already carries the prior: Ip enters as 1)
// fz (frozen importance): ps holds (da, sum_i gbv_i (beta v)_i) and the gate
// has no prior term.
__global__ __launch_bounds__(256) void bwd_gate_kernel(const float *ps, const void *dt, int dt_bf16,
                                                        const float *A, const float *Ip, int ipe, int fz, float *gdt,
                                                        float *gabh, float *gibh, int B, int T, int H, int nrb) {
    __shared__ float sh[2][4];
    const int bh = blockIdx.x, b = bh / H, h = bh % H;
    const size_t bth = (size_t)B * T * H;
    const float Ah = A[h], Iph = ipe ? 1.f : Ip[h];
    float accA = 0.f, accI = 0.f;
    for (int t = threadIdx.x; t < T; t += 256) {
        const size_t row = ((size_t)b * T + t) * H + h;
        // the row blocks' partials in order, 8 loads in flight at a time
        float da = 0.f, dc = 0.f;
        for (int r0 = 0; r0 < nrb; r0 += 8) {
            float2 x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = r0 + u < nrb ? r0 + u : nrb - 1;
                x[u] = *(const float2 *)(ps + ((size_t)r * bth + (size_t)bh * T + t) * 2);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (r0 + u < nrb) { da += x[u].x; dc += x[u].y; }
        }
        const float d = dt_bf16 ? (float)((const bf16_t *)dt)[row] : ((const float *)dt)[row];
        const float x = -Ah * d;
        const float al = expf(x), oma = -expm1f(x);
        const float u = fz ? -da : fmaf(Iph, dc, -da);
        gdt[row] = Ah * al * u;
        accA = fmaf(d * al, u, accA);
        accI = fz ? accI + dc : fmaf(oma, dc, accI);
    }
    accA = row16_sum(accA);
    accI = row16_sum(accI);
    accA += __shfl_xor(accA, 16, 64); accA += __shfl_xor(accA, 32, 64);
    accI += __shfl_xor(accI, 16, 64); accI += __shfl_xor(accI, 32, 64);
    if ((threadIdx.x & 63) == 0) { sh[0][threadIdx.x >> 6] = accA; sh[1][threadIdx.x >> 6] = accI; }
    __syncthreads();
    if (threadIdx.x == 0) {
        gabh[bh] = (sh[0][0] + sh[0][1]) + (sh[0][2] + sh[0][3]);
        gibh[bh] = (sh[1][0] + sh[1][1]) + (sh[1][2] + sh[1][3]);
    }
}

// gA, gI_prior per head: sums over the batch (plus the start state's share
// when it defaults to I_prior).  With a prior per entry only gA is written
// here (gI_prior comes from bwd_prior_kernel).
// fz: the frozen-importance prior gradient, -(1 / I_prior) sum gbv . (beta v).
__global__ __launch_bounds__(64) void bwd_head_kernel(const float *gabh, const float *gibh, const float *pI0,
                                                       const float *Ip, float *gA, float *gIp, int B, int H, int nrb,
                                                       int dflt, int ipe, int fz) {
    const int h = blockIdx.x * 64 + threadIdx.x;
    if (h >= H) return;
    float sa = 0.f, si = 0.f;
    for (int b = 0; b < B; ++b) {
        sa += gabh[(size_t)b * H + h];
        si += gibh[(size_t)b * H + h];
        if (dflt)
            for (int r = 0; r < nrb; ++r) si += pI0[((size_t)b * H + h) * nrb + r];
    }
    gA[h] = sa;
    if (fz) gIp[h] = -si / Ip[h];
    else if (!ipe) gIp[h] = si;
}

// Per-entry prior: gI_prior[h, i, j] = sum over the batch of the sequences'
// gradients (4 entries per thread).
__global__ __launch_bounds__(256) void bwd_prior_kernel(const float *pip, float *gIp, int B, size_t per_b) {
    const size_t n4 = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (4 * n4 >= per_b) return;
    float4 acc = *(const float4 *)(pip + 4 * n4);
    for (int b = 1; b < B; ++b) {
        const float4 x = *(const float4 *)(pip + (size_t)b * per_b + 4 * n4);
        acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
    }
    *(float4 *)(gIp + 4 * n4) = acc;
}

// ---------------------------------------------------------------------------
// block-diagonal precision (limited cross-key correlations), 2x2 blocks
// ---------------------------------------------------------------------------
//
// The Gaussian update of a value row (slides, backup frame "dropping
// precision correlations changes the mean", App. A.3-A.5) with the precision
// kept block-diagonal along the key axis, 2x2 blocks (the slides' closing
// question on limited cross-key correlations; a block of 1 is Eq. (5)).  In
// natural parameters h = P mu both stay affine:
//     P_t = alpha P_{t-1} + (1 - alpha) I_prior Id + beta_i blocks(k k^T)
//     h_t = alpha h_{t-1} + (beta_i v_i) k
// and the readout solves each 2x2 block: mu = P^{-1} h, y_i = sum_j mu_j q_j.
// The lane layout is the forward's (one row, DK/16 columns, which come in
// aligned 4-wide vectors, so a lane owns whole blocks).  Per block and token:
// 21 VALU + 1 v_rcp_f32 (10.5 VALU + 0.5 rcp per entry, against 6 + 1).
struct BdArgs {
    const void *q, *k, *v, *beta, *dt;
    const float *A, *Ip, *mu0, *P0;   // P0 / PT: [B, H, dv, dk/2, 2, 2]
    void *y;
    float *muT, *PT;
    float *ck;         // the training forward: the backward's checkpoints (else NULL)
    float *ck_sink;    // ... and one workgroup block that takes the stores past the sequence
    int B, T, H, dv, nwg, xcd_remap, nsb;
};

// A lane's block state: h for its KC columns, then per block the upper
// triangle of P ((p00, p01, p11) for 2x2 blocks, 10 entries for 4x4); a
// checkpoint pads it to whole float4s.
template <int DK, int BS> struct BdLane {
    static constexpr int kKC = LaneTile<DK>::kCols;
    static constexpr int kN = kKC + (BS == 2 ? 3 * (kKC / 2) : 10 * (kKC / 4));
    static constexpr int kNP = (kN + 3) / 4 * 4;
};
template <int DK> using Bd2Lane = BdLane<DK, 2>;

// A workgroup's checkpoint block: float4 i of thread tid at blk + 4 (i kThreads + tid).
template <int N, int NP>
__device__ inline void bd2_ck_store(float *blk, int tid, const float *x) {
#pragma unroll
    for (int i = 0; i < NP; i += 4)
        __builtin_nontemporal_store(f32x4{i < N ? x[i] : 0.f, i + 1 < N ? x[i + 1] : 0.f,
                                          i + 2 < N ? x[i + 2] : 0.f, i + 3 < N ? x[i + 3] : 0.f},
                                    (f32x4 *)(blk + 4 * ((i / 4) * kThreads + tid)));
}
template <int N, int NP>
__device__ inline void bd2_ck_load(const float *blk, int tid, float *x) {
#pragma unroll
    for (int i = 0; i < NP; i += 4) {
        const f32x4 v = __builtin_nontemporal_load((const f32x4 *)(blk + 4 * ((i / 4) * kThreads + tid)));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (i + j < N) x[i + j] = v[j];
    }
}


// CKPT (the training forward): the lane's state before the chunk's tokens 0
// and 8 is stored as the backward's checkpoint at ck_a and ck_b (a discard
// block where the sequence has no such sub-block), unconditionally, so the
// token loop stays one straight-line block.
template <int DK, int C, typename TOut, bool CKPT = false>
__device__ inline void bd2_chunk(const float *buf, int left, float *h, float *p00, float *p01, float *p11,
                                 int row_local, int g, TOut *yrow, size_t ystride,
                                 float *ck_a = nullptr, float *ck_b = nullptr) {
    using LT = LaneTile<DK>;
    using L = BdLane<DK, 2>;
    static_assert(!CKPT || (C == 16 && kGroup == 2 * kSB), "the checkpointing forward runs chunk 16");
    const float *cbase = buf + LT::col(g, 0, 0);
    const float *rbase = buf + C * Stage<DK>::kColFloats + 2 * row_local;
    int goff = C * (Stage<DK>::kColFloats + Stage<DK>::kRowFloats);
    asm volatile("" : "+v"(goff));
    const float *gbase = buf + goff;
#pragma unroll 1
    for (int grp = 0; grp < C / kGroup; ++grp) {
        const float *cg = cbase + grp * kGroup * Stage<DK>::kColFloats;
        const float *rg = rbase + grp * kGroup * Stage<DK>::kRowFloats;
        const float *gg = gbase + grp * kGroup * 2;
        float part[kGroup];
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            if (CKPT && u % kSB == 0) {
                float st[L::kN];
#pragma unroll
                for (int x = 0; x < LT::kCols; ++x) st[x] = h[x];
#pragma unroll
                for (int pb = 0; pb < LT::kCols / 2; ++pb) {
                    st[LT::kCols + 3 * pb] = p00[pb];
                    st[LT::kCols + 3 * pb + 1] = p01[pb];
                    st[LT::kCols + 3 * pb + 2] = p11[pb];
                }
                bd2_ck_store<L::kN, L::kNP>(u == 0 ? ck_a : ck_b, threadIdx.x, st);
            }
            const float2 gc = *(const float2 *)(gg + 2 * u);                          // alpha, c
            const float2 rb = *(const float2 *)(rg + u * Stage<DK>::kRowFloats);      // beta, beta*v
            const float *ct = cg + u * Stage<DK>::kColFloats;
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < LT::kNVec; ++m) {
                float kk[LT::kVec], k2[LT::kVec], qq[LT::kVec];
                const int c0 = kLanesPerRow * LT::kVec * m;
                vecf<LT::kVec>::ld(ct + c0, kk);
                vecf<LT::kVec>::ld(ct + DK + c0, k2);
                vecf<LT::kVec>::ld(ct + 2 * DK + c0, qq);
#pragma unroll
                for (int e = 0; e < LT::kVec; e += 2) {
                    const int s = m * LT::kVec + e, pb = s / 2;
                    p00[pb] = fmaf(gc.x, p00[pb], fmaf(rb.x, k2[e], gc.y));
                    p11[pb] = fmaf(gc.x, p11[pb], fmaf(rb.x, k2[e + 1], gc.y));
                    p01[pb] = fmaf(gc.x, p01[pb], rb.x * (kk[e] * kk[e + 1]));
                    h[s] = fmaf(gc.x, h[s], rb.y * kk[e]);
                    h[s + 1] = fmaf(gc.x, h[s + 1], rb.y * kk[e + 1]);
                    const float r = __builtin_amdgcn_rcpf(fmaf(p00[pb], p11[pb], -(p01[pb] * p01[pb])));
                    const float m0 = fmaf(p11[pb], h[s], -(p01[pb] * h[s + 1])) * r;
                    const float m1 = fmaf(p00[pb], h[s + 1], -(p01[pb] * h[s])) * r;
                    acc = fmaf(m0, qq[e], acc);
                    acc = fmaf(m1, qq[e + 1], acc);
                }
            }
            part[u] = acc;
        }
        const float yv = row16_transpose_sum(part, g);
        const int tt = grp * kGroup + g;
        if (tt < left)
            yrow[(size_t)tt * ystride] = io<TOut>::from_f32(yv);
    }
}

template <int DK, int C, typename TIn, typename TOut, bool CKPT = false>
__global__ __launch_bounds__(kThreads) void bd2_fwd_kernel(BdArgs a) {
    using LT = LaneTile<DK>;
    static_assert(LT::kVec % 2 == 0, "a lane's columns must hold whole 2-blocks");
    constexpr int KC = LT::kCols, KB = KC / 2;
    extern __shared__ float lds[];
    float *buf0 = lds;
    float *buf1 = lds + C * Stage<DK>::kTokFloats;
    const int rb_per_head = a.dv / kRowsPerWG;
    int wg = blockIdx.x;
    if (a.xcd_remap) {
        const int per_xcd = a.nwg / 8;
        wg = (wg % 8) * per_xcd + wg / 8;
    }
    const int bh = wg / rb_per_head;
    const int row0 = (wg % rb_per_head) * kRowsPerWG;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane & (kLanesPerRow - 1);
    const int row_local = wave * kRowsPerWave + (lane >> 4);
    const int row = row0 + row_local;
    const float A = a.A[h], Ip = a.Ip[h];

    // state: h = P mu per entry, (p00, p01, p11) per 2-block
    float hv[KC], p00[KB], p01[KB], p11[KB];
    const size_t srow = ((size_t)bh * a.dv + row) * DK;      // entry (b, h, row, 0)
#pragma unroll
    for (int m = 0; m < LT::kNVec; ++m)
#pragma unroll
        for (int e = 0; e < LT::kVec; e += 2) {
            const int s = m * LT::kVec + e, pb = s / 2;
            const int col = LT::col(g, m, e);                 // even: the block's first column
            if (a.mu0) {
                const float4 P = *(const float4 *)(a.P0 + (srow + col) * 2);   // block (col / 2): 2x2
                const float m0 = a.mu0[srow + col], m1 = a.mu0[srow + col + 1];
                p00[pb] = P.x; p01[pb] = P.y; p11[pb] = P.w;
                hv[s] = fmaf(P.x, m0, P.y * m1);
                hv[s + 1] = fmaf(P.y, m0, P.w * m1);
            } else {
                p00[pb] = Ip; p01[pb] = 0.f; p11[pb] = Ip;
                hv[s] = 0.f; hv[s + 1] = 0.f;
            }
        }

    const size_t seq = (size_t)b * a.T * a.H + h;
    const TIn *kseq = (const TIn *)a.k + seq * DK;
    const TIn *qseq = (const TIn *)a.q + seq * DK;
    const TIn *vseq = (const TIn *)a.v + seq * a.dv + row0;
    const TIn *bseq = (const TIn *)a.beta + seq * a.dv + row0;
    const TIn *dseq = (const TIn *)a.dt + seq;
    const size_t kq_tok = (size_t)a.H * DK, vb_tok = (size_t)a.H * a.dv;
    const size_t ystride = (size_t)a.H * a.dv;
    TOut *ybase = (TOut *)a.y + seq * a.dv + row;
    const size_t ck_stride = CKPT ? (size_t)rb_per_head * kThreads * BdLane<DK, 2>::kNP : 0;
    float *ckb = CKPT ? a.ck + ((size_t)bh * a.nsb * rb_per_head + wg % rb_per_head) *
                                   (kThreads * BdLane<DK, 2>::kNP)
                      : nullptr;
    // sub-block sb's checkpoint block, or the discard block past the sequence
    auto ck_at = [&](int sb) { return !CKPT ? nullptr : sb < a.nsb ? ckb + (size_t)sb * ck_stride : a.ck_sink; };
    const int nchunks = (a.T + C - 1) / C;
    Stager<DK, C, TIn, true> st;
    if (nchunks > 0) {
        st.load(kseq, qseq, vseq, bseq, dseq, a.T, a.H, a.dv, tid);
        st.commit(buf0, A, Ip, tid, false);
        __syncthreads();
    }
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C;
        const bool more = c + 1 < nchunks;
        if (more) {
            const size_t tn = (size_t)(t0 + C);
            st.load(kseq + tn * kq_tok, qseq + tn * kq_tok, vseq + tn * vb_tok, bseq + tn * vb_tok,
                    dseq + tn * a.H, a.T - (t0 + C), a.H, a.dv, tid);
        }
        bd2_chunk<DK, C, TOut, CKPT>((c & 1) ? buf1 : buf0, a.T - t0, hv, p00, p01, p11, row_local, g,
                                     ybase + (size_t)t0 * ystride, ystride, ck_at(t0 / kSB), ck_at(t0 / kSB + 1));
        if (more) st.commit((c & 1) ? buf0 : buf1, A, Ip, tid, false);
        __syncthreads();
    }
    if (a.muT) {
#pragma unroll
        for (int m = 0; m < LT::kNVec; ++m)
#pragma unroll
            for (int e = 0; e < LT::kVec; e += 2) {
                const int s = m * LT::kVec + e, pb = s / 2;
                const int col = LT::col(g, m, e);
                float m0, m1;
                if (a.T == 0 && a.mu0) {
                    m0 = a.mu0[srow + col]; m1 = a.mu0[srow + col + 1];   // copied through exactly
                } else {
                    const float det = fmaf(p00[pb], p11[pb], -(p01[pb] * p01[pb]));
                    m0 = fmaf(p11[pb], hv[s], -(p01[pb] * hv[s + 1])) / det;
                    m1 = fmaf(p00[pb], hv[s + 1], -(p01[pb] * hv[s])) / det;
                }
                a.muT[srow + col] = m0;
                a.muT[srow + col + 1] = m1;
                *(float4 *)(a.PT + (srow + col) * 2) = make_float4(p00[pb], p01[pb], p01[pb], p11[pb]);
            }
    }
}

// ---------------------------------------------------------------------------
// block-diagonal precision (2x2 blocks): backward
// ---------------------------------------------------------------------------
//
// Reverse mode through the 2x2 block update above, per value row and key
// block, walking t = T-1 .. 0 with (G_h, G_P) the adjoints of (h_t, P_t).
// Every use of P is a symmetric form, so only S = (G_P + G_P^T) / 2 matters
// and a block carries it as (s00, s01, s11).  Per token and block:
//   readout  mu = P^-1 h, w = P^-1 (gy_i q_b):  gq_b += gy_i mu,
//            G_h += w,  S -= (w mu^T + mu w^T) / 2
//   update   gk_b += (beta v)_i G_h + 2 beta_i S k_b,
//            gbv_i += G_h . k_b,  gb_i += k_b^T S k_b (beta's precision term),
//            da += G_h . h_{t-1} + <S, P_{t-1}>,  dc += tr S,
//            then (G_h, S) *= alpha_t.
// These are the exact backward's four row sums and two column sums, so its
// finishing kernels (gq, gk; gdt; gA, gI_prior) serve unchanged.  The final
// state's adjoint is G_h = P_T^-1 gmuT, S = sym(gPT) - sym(G_h mu_T^T); at the
// start h_0 = P_0 mu_0 gives gmu0 = P_0 G_h and gP0 = S + sym(G_h mu0^T)
// (the gradient for a symmetric P0), and the default start (mu0 = 0,
// P_0 = I_prior Id) adds tr S to gI_prior.
//
// Passes: bd_ckpt_kernel stores (h, P) before every 8th token; bd2_bwd_kernel
// has bwd_kernel's structure (halves of 4 tokens replayed from the
// checkpoint into registers, walked in reverse) with the step above.


// The lane's start state: from (mu0, P0) when given (P0's upper triangle),
// else mu0 = 0 and P0 = I_prior Id.  srow: entry (b, h, row, 0).
template <int DK>
__device__ inline void bd2_start(const float *mu0, const float *P0, size_t srow, int g, float Ip, float *st) {
    using LT = LaneTile<DK>;
    constexpr int KC = LT::kCols;
#pragma unroll
    for (int m = 0; m < LT::kNVec; ++m)
#pragma unroll
        for (int e = 0; e < LT::kVec; e += 2) {
            const int s = m * LT::kVec + e;
            float *p = st + KC + 3 * (s / 2);
            const int col = LT::col(g, m, e);
            if (mu0) {
                const float4 P = *(const float4 *)(P0 + (srow + col) * 2);
                const float m0 = mu0[srow + col], m1 = mu0[srow + col + 1];
                p[0] = P.x; p[1] = P.y; p[2] = P.w;
                st[s] = fmaf(P.x, m0, P.y * m1);
                st[s + 1] = fmaf(P.y, m0, P.w * m1);
            } else {
                p[0] = Ip; p[1] = 0.f; p[2] = Ip;
                st[s] = 0.f; st[s + 1] = 0.f;
            }
        }
}

// One token's update of the lane's blocks (bd2_chunk's operations).  ct: the
// token's staged k at ct[c], k^2 at ct[DK + c], from the lane's first column.
template <int DK>
__device__ inline void bd2_update(const float *ct, float alpha, float c, float beta, float bv, float *st) {
    using LT = LaneTile<DK>;
    constexpr int KC = LT::kCols;
#pragma unroll
    for (int m = 0; m < LT::kNVec; ++m) {
        float kk[LT::kVec], k2[LT::kVec];
        const int c0 = kLanesPerRow * LT::kVec * m;
        vecf<LT::kVec>::ld(ct + c0, kk);
        vecf<LT::kVec>::ld(ct + DK + c0, k2);
#pragma unroll
        for (int e = 0; e < LT::kVec; e += 2) {
            const int s = m * LT::kVec + e;
            float *p = st + KC + 3 * (s / 2);
            p[0] = fmaf(alpha, p[0], fmaf(beta, k2[e], c));
            p[2] = fmaf(alpha, p[2], fmaf(beta, k2[e + 1], c));
            p[1] = fmaf(alpha, p[1], beta * (kk[e] * kk[e + 1]));
            st[s] = fmaf(alpha, st[s], bv * kk[e]);
            st[s + 1] = fmaf(alpha, st[s + 1], bv * kk[e + 1]);
        }
    }
}

struct BdBwdArgs {
    const void *q, *k, *v, *beta, *dt, *gy;
    const float *A, *Ip, *mu0, *P0, *gmuT, *gPT;    // P0, gPT: [B, H, dv, dk/2, 2, 2]
    float *gv, *gbeta, *gmu0, *gP0;
    float *ck;         // [B*H][T/8][dv/16][lane state]: (h, P) before every 8th token
    float *pqk, *ps, *pI0;   // bwd_kernel's partials, same layouts
    int B, T, H, dv, nsb, nwg, xcd_remap;
    int ck_saved;      // the training forward stored the checkpoints already
};

// A sub-block's outputs once its (gq, gk) column sums are in red and its row
// sums (gbv, gb, da, dc) in rs: the row block's (gq, gk) partials summed over
// the 4 waves, gv = gbv beta and gbeta = gbv v + gb per (token, row), and the
// row block's (da, dc) partials per token.
template <int DK>
__device__ inline void bd_bwd_epilogue(const BdBwdArgs &a, const float *cur, const float *red, const float *rs,
                                       int tid, int t0, int rb, int bh, int row0, size_t seq0, size_t bth) {
    using S = BwdStage<DK>;
    for (int n = 4 * tid; n < kSB * 2 * DK; n += 4 * kThreads) {
        const int e = n / (2 * DK), c = n % (2 * DK);
        const float *r0 = red + e * kWaves * 2 * DK + c;
        const float4 v0 = *(const float4 *)r0, v1 = *(const float4 *)(r0 + 2 * DK);
        const float4 v2 = *(const float4 *)(r0 + 4 * DK), v3 = *(const float4 *)(r0 + 6 * DK);
        if (t0 + e < a.T)
            *(float4 *)(a.pqk + ((size_t)rb * bth + seq0 + (size_t)(t0 + e) * a.H) * 2 * DK + c) =
                make_float4((v0.x + v1.x) + (v2.x + v3.x), (v0.y + v1.y) + (v2.y + v3.y),
                            (v0.z + v1.z) + (v2.z + v3.z), (v0.w + v1.w) + (v2.w + v3.w));
    }
    if (tid < kSB * kRowsPerWG) {
        const int e = tid / kRowsPerWG, r = tid % kRowsPerWG;
        const float gbv = rs[(e * 4 + 0) * kRowsPerWG + r], gb = rs[(e * 4 + 1) * kRowsPerWG + r];
        const float4 rw = *(const float4 *)(cur + S::kRows + e * S::kRowFloats + 4 * r);
        if (t0 + e < a.T) {
            const size_t o = (seq0 + (size_t)(t0 + e) * a.H) * a.dv + row0 + r;
            a.gv[o] = gbv * rw.x;
            a.gbeta[o] = fmaf(gbv, rw.z, gb);
        }
    } else if (tid < kSB * kRowsPerWG + 2 * kSB) {
        const int u = tid - kSB * kRowsPerWG, e = u % kSB, qd = u / kSB;
        const float *src = rs + (e * 4 + 2 + qd) * kRowsPerWG;
        float v = 0.f;
#pragma unroll
        for (int r = 0; r < kRowsPerWG; ++r) v += src[r];
        if (t0 + e < a.T) a.ps[((size_t)rb * bth + (size_t)bh * a.T + t0 + e) * 2 + qd] = v;
    }
}

// The workgroup's sum of the lanes' x into pI0[slot] (rs: 4 floats of scratch LDS).
__device__ inline void bd_bwd_trace_partial(const BdBwdArgs &a, float x, float *rs, int tid, size_t slot) {
    x = row16_sum(x);
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    __syncthreads();
    if ((tid & 63) == 0) rs[tid >> 6] = x;
    __syncthreads();
    if (tid == 0) a.pI0[slot] = (rs[0] + rs[1]) + (rs[2] + rs[3]);
}

// One token of the reverse walk for the lane's blocks: St the state after the
// token, Sp before it.  Updates (Gh, GS), returns the lane's row partials of
// (gbv, gb, da, dc) and writes the wave's (gq, gk) column sums to red as
// bwd_reverse_token does.
template <int DK>
__device__ inline void bd2_reverse_token(const float *buf, int e, const float *St, const float *Sp, float *Gh,
                                         float *GS, int row_local, int g, int lane, float *red,
                                         float &cbv, float &cb, float &s1, float &s2) {
    using LT = LaneTile<DK>;
    using S = BwdStage<DK>;
    constexpr int KC = LT::kCols;
    const float alpha = buf[S::kGate + 2 * e];
    const float4 rw = *(const float4 *)(buf + S::kRows + e * S::kRowFloats + 4 * row_local);
    const float b2 = 2.f * rw.x, bv = rw.y, gy = rw.w;
    const float *ct = buf + e * S::kColFloats + LT::col(g, 0, 0);
    float dq[KC], dk[KC];
    cbv = 0.f; cb = 0.f; s1 = 0.f; s2 = 0.f;
#pragma unroll
    for (int m = 0; m < LT::kNVec; ++m) {
        float kk[LT::kVec], qq[LT::kVec];
        const int c0 = kLanesPerRow * LT::kVec * m;
        vecf<LT::kVec>::ld(ct + c0, kk);
        vecf<LT::kVec>::ld(ct + 2 * DK + c0, qq);
#pragma unroll
        for (int x = 0; x < LT::kVec; x += 2) {
            const int s = m * LT::kVec + x;
            const float *p = St + KC + 3 * (s / 2), *pp = Sp + KC + 3 * (s / 2);
            float *gs = GS + 3 * (s / 2);
            const float r = __builtin_amdgcn_rcpf(fmaf(p[0], p[2], -(p[1] * p[1])));
            const float m0 = fmaf(p[2], St[s], -(p[1] * St[s + 1])) * r;
            const float m1 = fmaf(p[0], St[s + 1], -(p[1] * St[s])) * r;
            const float g0 = gy * qq[x], g1 = gy * qq[x + 1];
            const float w0 = fmaf(p[2], g0, -(p[1] * g1)) * r;
            const float w1 = fmaf(p[0], g1, -(p[1] * g0)) * r;
            dq[s] = gy * m0;
            dq[s + 1] = gy * m1;
            Gh[s] += w0;
            Gh[s + 1] += w1;
            gs[0] = fmaf(-w0, m0, gs[0]);
            gs[2] = fmaf(-w1, m1, gs[2]);
            gs[1] = fmaf(-0.5f, fmaf(w0, m1, w1 * m0), gs[1]);
            const float k0 = kk[x], k1 = kk[x + 1];
            const float sk0 = fmaf(gs[0], k0, gs[1] * k1), sk1 = fmaf(gs[1], k0, gs[2] * k1);
            dk[s] = fmaf(Gh[s], bv, b2 * sk0);
            dk[s + 1] = fmaf(Gh[s + 1], bv, b2 * sk1);
            cbv = fmaf(Gh[s], k0, fmaf(Gh[s + 1], k1, cbv));
            cb = fmaf(sk0, k0, fmaf(sk1, k1, cb));
            s1 = fmaf(Gh[s], Sp[s], fmaf(Gh[s + 1], Sp[s + 1], s1));
            s1 = fmaf(gs[0], pp[0], fmaf(gs[2], pp[2], fmaf(2.f * gs[1], pp[1], s1)));
            s2 += gs[0] + gs[2];
            Gh[s] *= alpha;
            Gh[s + 1] *= alpha;
            gs[0] *= alpha;
            gs[1] *= alpha;
            gs[2] *= alpha;
        }
    }
    bwd_scatter_qk<DK>(dq, dk, lane, g, red);
}

template <int DK, typename TIn, typename TG>
// Two workgroups per CU (two waves per SIMD, 256 registers per lane at most):
// the next checkpoint is loaded into ckS once ckS is dead rather than into a
// prefetch copy, which is what keeps the lane within that budget.
__global__ __launch_bounds__(kThreads, 2) void bd2_bwd_kernel(BdBwdArgs a) {
    using LT = LaneTile<DK>;
    using S = BwdStage<DK>;
    using L = Bd2Lane<DK>;
    constexpr int KC = LT::kCols, KB = KC / 2, N = L::kN;
    extern __shared__ float lds[];
    float *red = lds + S::kRed;
    float *rs = lds + S::kRs;

    const int rb_per_head = a.dv / kRowsPerWG;
    int wg = blockIdx.x;
    if (a.xcd_remap) {
        const int per_xcd = a.nwg / 8;
        wg = (wg % 8) * per_xcd + wg / 8;
    }
    const int bh = wg / rb_per_head;
    const int rb = wg % rb_per_head;
    const int row0 = rb * kRowsPerWG;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane & (kLanesPerRow - 1);
    const int row_local = wave * kRowsPerWave + (lane >> 4);
    const float A = a.A[h], Ip = a.Ip[h];
    const size_t srow = ((size_t)bh * a.dv + row0 + row_local) * DK;
    const size_t seq0 = (size_t)b * a.T * a.H + h;
    const size_t bth = (size_t)a.B * a.T * a.H;
    const size_t kq_tok = (size_t)a.H * DK, vb_tok = (size_t)a.H * a.dv;

    float Gh[KC], GS[3 * KB];
    // the final state's adjoint from (gmuT, gPT), given the final state st
    auto final_adjoint = [&](const float *st) {
#pragma unroll
        for (int m = 0; m < LT::kNVec; ++m)
#pragma unroll
            for (int x = 0; x < LT::kVec; x += 2) {
                const int s = m * LT::kVec + x;
                const size_t o = srow + LT::col(g, m, x);
                const float *p = st + KC + 3 * (s / 2);
                const float gm0 = a.gmuT ? a.gmuT[o] : 0.f, gm1 = a.gmuT ? a.gmuT[o + 1] : 0.f;
                const float4 gp = a.gPT ? *(const float4 *)(a.gPT + o * 2) : make_float4(0.f, 0.f, 0.f, 0.f);
                const float det = fmaf(p[0], p[2], -(p[1] * p[1]));
                const float mT0 = fmaf(p[2], st[s], -(p[1] * st[s + 1])) / det;
                const float mT1 = fmaf(p[0], st[s + 1], -(p[1] * st[s])) / det;
                const float w0 = fmaf(p[2], gm0, -(p[1] * gm1)) / det;
                const float w1 = fmaf(p[0], gm1, -(p[1] * gm0)) / det;
                float *gs = GS + 3 * (s / 2);
                Gh[s] = w0;
                Gh[s + 1] = w1;
                gs[0] = fmaf(-w0, mT0, gp.x);
                gs[2] = fmaf(-w1, mT1, gp.w);
                gs[1] = 0.5f * ((gp.y + gp.z) - fmaf(w0, mT1, w1 * mT0));
            }
    };

    if (a.nsb == 0) {
        // T = 0: mu_T = mu_0 and P_T = P_0 are copied through, so are their gradients
#pragma unroll
        for (int m = 0; m < LT::kNVec; ++m)
#pragma unroll
            for (int x = 0; x < LT::kVec; x += 2) {
                const int s = m * LT::kVec + x;
                const size_t o = srow + LT::col(g, m, x);
                const float4 gp = a.gPT ? *(const float4 *)(a.gPT + o * 2) : make_float4(0.f, 0.f, 0.f, 0.f);
                float *gs = GS + 3 * (s / 2);
                gs[0] = gp.x; gs[1] = 0.5f * (gp.y + gp.z); gs[2] = gp.w;
                if (a.gmu0) {
                    a.gmu0[o] = a.gmuT ? a.gmuT[o] : 0.f;
                    a.gmu0[o + 1] = a.gmuT ? a.gmuT[o + 1] : 0.f;
                }
                if (a.gP0) *(float4 *)(a.gP0 + o * 2) = make_float4(gs[0], gs[1], gs[1], gs[2]);
            }
    } else {
        const size_t ck_stride = (size_t)rb_per_head * kThreads * L::kNP;
        const float *ckb = a.ck + ((size_t)bh * a.nsb * rb_per_head + rb) * (kThreads * L::kNP);
        const TIn *kseq = (const TIn *)a.k + seq0 * DK;
        const TIn *qseq = (const TIn *)a.q + seq0 * DK;
        const TIn *vseq = (const TIn *)a.v + seq0 * a.dv + row0;
        const TIn *bseq = (const TIn *)a.beta + seq0 * a.dv + row0;
        const TG *gseq = (const TG *)a.gy + seq0 * a.dv + row0;
        const TIn *dseq = (const TIn *)a.dt + seq0;
        BwdStager<DK, TIn, TG> st;
        {
            const size_t tn = (size_t)(a.nsb - 1) * kSB;
            st.load(kseq + tn * kq_tok, qseq + tn * kq_tok, vseq + tn * vb_tok, bseq + tn * vb_tok,
                    gseq + tn * vb_tok, dseq + tn * a.H, a.T - (int)tn, a.H, a.dv, tid);
            st.commit(lds + ((a.nsb - 1) & 1) * S::kFloats, A, Ip, tid, false);
        }
        float ckS[N];
        bd2_ck_load<N, L::kNP>(ckb + (size_t)(a.nsb - 1) * ck_stride, tid, ckS);
        __syncthreads();

        for (int sb = a.nsb - 1; sb >= 0; --sb) {
            const float *cur = lds + (sb & 1) * S::kFloats;
            const int t0 = sb * kSB;
            // the checkpoint (loaded at the end of the previous sub-block) is
            // waited for before the next loads go out, not behind them
            regs_ready<N>(ckS);
            if (sb > 0) {
                const size_t tn = (size_t)(t0 - kSB);
                st.load(kseq + tn * kq_tok, qseq + tn * kq_tok, vseq + tn * vb_tok, bseq + tn * vb_tok,
                        gseq + tn * vb_tok, dseq + tn * a.H, a.T - (int)tn, a.H, a.dv, tid);
            }
            auto replay = [&](int e, float *x) {
                const float2 gc = *(const float2 *)(cur + S::kGate + 2 * e);
                const float2 rw = *(const float2 *)(cur + S::kRows + e * S::kRowFloats + 4 * row_local);
                bd2_update<DK>(cur + e * S::kColFloats + LT::col(g, 0, 0), gc.x, gc.y, rw.x, rw.y, x);
            };
            float xS[4][N];
            float acc[16];      // this half's row partials: gbv, gb, da, dc of its 4 tokens
            // upper half: tokens 4..7, replayed from the checkpoint
            float mS[N];
#pragma unroll
            for (int i = 0; i < N; ++i) mS[i] = ckS[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) replay(e, mS);
#pragma unroll
            for (int e = 4; e < 8; ++e) {
                const float *pv = e == 4 ? mS : xS[e > 4 ? e - 5 : 0];
#pragma unroll
                for (int i = 0; i < N; ++i) xS[e - 4][i] = pv[i];
                replay(e, xS[e - 4]);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (sb == a.nsb - 1) final_adjoint(xS[3]);   // tokens past T are neutral
#pragma unroll
            for (int e = 7; e >= 4; --e) {
                bd2_reverse_token<DK>(cur, e, xS[e - 4], e == 4 ? mS : xS[e > 4 ? e - 5 : 0], Gh, GS, row_local,
                                      g, lane, red + (e * kWaves + wave) * 2 * DK,
                                      acc[e - 4], acc[e], acc[e + 4], acc[e + 8]);
                __builtin_amdgcn_sched_barrier(0);
            }
            bwd_row_sums(acc, g, rs + 4 * 4 * kRowsPerWG + row_local);
            if (sb > 0) st.ready();    // half a sub-block after the loads, before any store
            // lower half: tokens 0..3
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float *pv = e == 0 ? ckS : xS[e > 0 ? e - 1 : 0];
#pragma unroll
                for (int i = 0; i < N; ++i) xS[e][i] = pv[i];
                replay(e, xS[e]);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int e = 3; e >= 0; --e) {
                bd2_reverse_token<DK>(cur, e, xS[e], e == 0 ? ckS : xS[e > 0 ? e - 1 : 0], Gh, GS, row_local,
                                      g, lane, red + (e * kWaves + wave) * 2 * DK,
                                      acc[e], acc[e + 4], acc[e + 8], acc[e + 12]);
                __builtin_amdgcn_sched_barrier(0);
            }
            bwd_row_sums(acc, g, rs + row_local);
            // the next checkpoint, into ckS now that token 0's reverse step has used it
            if (sb > 0) bd2_ck_load<N, L::kNP>(ckb + (size_t)(sb - 1) * ck_stride, tid, ckS);
            if (sb > 0) st.commit(lds + ((sb - 1) & 1) * S::kFloats, A, Ip, tid, false);
            __syncthreads();
            bd_bwd_epilogue<DK>(a, cur, red, rs, tid, t0, rb, bh, row0, seq0, bth);
            __syncthreads();
        }
        // the start state h_0 = P_0 mu_0
#pragma unroll
        for (int m = 0; m < LT::kNVec; ++m)
#pragma unroll
            for (int x = 0; x < LT::kVec; x += 2) {
                const int s = m * LT::kVec + x;
                const size_t o = srow + LT::col(g, m, x);
                float *gs = GS + 3 * (s / 2);
                float4 P = make_float4(Ip, 0.f, 0.f, Ip);
                float m0 = 0.f, m1 = 0.f;
                if (a.mu0) {
                    P = *(const float4 *)(a.P0 + o * 2);
                    m0 = a.mu0[o];
                    m1 = a.mu0[o + 1];
                }
                if (a.gmu0) {
                    a.gmu0[o] = fmaf(P.x, Gh[s], P.y * Gh[s + 1]);
                    a.gmu0[o + 1] = fmaf(P.y, Gh[s], P.w * Gh[s + 1]);
                }
                gs[0] = fmaf(Gh[s], m0, gs[0]);
                gs[2] = fmaf(Gh[s + 1], m1, gs[2]);
                gs[1] = fmaf(0.5f, fmaf(Gh[s], m1, Gh[s + 1] * m0), gs[1]);
                if (a.gP0) *(float4 *)(a.gP0 + o * 2) = make_float4(gs[0], gs[1], gs[1], gs[2]);
            }
    }
    // this row block's sum of tr(gP0) (the default start P_0 = I_prior Id feeds gI_prior)
    float gs = 0.f;
#pragma unroll
    for (int j = 0; j < KB; ++j) gs += GS[3 * j] + GS[3 * j + 2];
    bd_bwd_trace_partial(a, gs, rs, tid, bh * rb_per_head + rb);
}

// ---------------------------------------------------------------------------
// block-diagonal precision, 4x4 blocks
// ---------------------------------------------------------------------------
//
// The same update with blocks of 4 adjacent key channels (a lane's aligned
// 4-wide column vector is one block, so d_k in {64, 128}).  A block keeps its
// natural parameter h (4) and the upper triangle of P (10); the readout solves
// P mu = h by Cholesky, P = L L^T, with 4 v_rsq_f32 for the diagonal of L^-1.
// Per block and token: 34 VALU for the update, 36 VALU + 4 rsq for the solve,
// 4 for the readout.

// Solve P x = h for a symmetric positive definite 4x4 P given by its upper
// triangle p = (p00 p01 p02 p03 p11 p12 p13 p22 p23 p33).
// The factor: r_i = 1 / L_ii and the strictly lower part of L.
struct Chol4 {
    float r0, r1, r2, r3, l10, l20, l30, l21, l31, l32;
};
__device__ inline Chol4 spd4_factor(const float *p) {
    Chol4 f;
    f.r0 = __builtin_amdgcn_rsqf(p[0]);
    f.l10 = p[1] * f.r0; f.l20 = p[2] * f.r0; f.l30 = p[3] * f.r0;
    f.r1 = __builtin_amdgcn_rsqf(fmaf(-f.l10, f.l10, p[4]));
    f.l21 = fmaf(-f.l20, f.l10, p[5]) * f.r1;
    f.l31 = fmaf(-f.l30, f.l10, p[6]) * f.r1;
    f.r2 = __builtin_amdgcn_rsqf(fmaf(-f.l21, f.l21, fmaf(-f.l20, f.l20, p[7])));
    f.l32 = fmaf(-f.l31, f.l21, fmaf(-f.l30, f.l20, p[8])) * f.r2;
    f.r3 = __builtin_amdgcn_rsqf(fmaf(-f.l32, f.l32, fmaf(-f.l31, f.l31, fmaf(-f.l30, f.l30, p[9]))));
    return f;
}
// L z = h, then L^T x = z.
__device__ inline void spd4_apply(const Chol4 &f, const float *h, float *x) {
    const float z0 = h[0] * f.r0;
    const float z1 = fmaf(-f.l10, z0, h[1]) * f.r1;
    const float z2 = fmaf(-f.l21, z1, fmaf(-f.l20, z0, h[2])) * f.r2;
    const float z3 = fmaf(-f.l32, z2, fmaf(-f.l31, z1, fmaf(-f.l30, z0, h[3]))) * f.r3;
    x[3] = z3 * f.r3;
    x[2] = fmaf(-f.l32, x[3], z2) * f.r2;
    x[1] = fmaf(-f.l31, x[3], fmaf(-f.l21, x[2], z1)) * f.r1;
    x[0] = fmaf(-f.l30, x[3], fmaf(-f.l20, x[2], fmaf(-f.l10, x[1], z0))) * f.r0;
}
__device__ inline void spd4_solve(const float *p, const float *h, float *x) { spd4_apply(spd4_factor(p), h, x); }

// One token's update of a 4-block: P = alpha P + c Id + beta k k^T, h = alpha h + (beta v) k.
__device__ inline void bd4_update(float *p, float *hh, const float *kk, const float *k2, float alpha, float c,
                                  float bt, float bv) {
    p[0] = fmaf(alpha, p[0], fmaf(bt, k2[0], c));
    p[4] = fmaf(alpha, p[4], fmaf(bt, k2[1], c));
    p[7] = fmaf(alpha, p[7], fmaf(bt, k2[2], c));
    p[9] = fmaf(alpha, p[9], fmaf(bt, k2[3], c));
    p[1] = fmaf(alpha, p[1], bt * (kk[0] * kk[1]));
    p[2] = fmaf(alpha, p[2], bt * (kk[0] * kk[2]));
    p[3] = fmaf(alpha, p[3], bt * (kk[0] * kk[3]));
    p[5] = fmaf(alpha, p[5], bt * (kk[1] * kk[2]));
    p[6] = fmaf(alpha, p[6], bt * (kk[1] * kk[3]));
    p[8] = fmaf(alpha, p[8], bt * (kk[2] * kk[3]));
#pragma unroll
    for (int e = 0; e < 4; ++e) hh[e] = fmaf(alpha, hh[e], bv * kk[e]);
}

template <int DK, int C, typename TOut, bool CKPT = false>
__device__ inline void bd4_chunk(const float *buf, int left, float *h, float (*P)[10], int row_local, int g,
                                 TOut *yrow, size_t ystride, float *ck_a = nullptr, float *ck_b = nullptr) {
    using LT = LaneTile<DK>;
    using L = BdLane<DK, 4>;
    static_assert(!CKPT || (C == 16 && kGroup == 2 * kSB), "the checkpointing forward runs chunk 16");
    const float *cbase = buf + LT::col(g, 0, 0);
    const float *rbase = buf + C * Stage<DK>::kColFloats + 2 * row_local;
    int goff = C * (Stage<DK>::kColFloats + Stage<DK>::kRowFloats);
    asm volatile("" : "+v"(goff));
    const float *gbase = buf + goff;
#pragma unroll 1
    for (int grp = 0; grp < C / kGroup; ++grp) {
        const float *cg = cbase + grp * kGroup * Stage<DK>::kColFloats;
        const float *rg = rbase + grp * kGroup * Stage<DK>::kRowFloats;
        const float *gg = gbase + grp * kGroup * 2;
        float part[kGroup];
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            if (CKPT && u % kSB == 0) {
                float st[L::kN];
#pragma unroll
                for (int x = 0; x < LT::kCols; ++x) st[x] = h[x];
#pragma unroll
                for (int mb = 0; mb < LT::kNVec; ++mb)
#pragma unroll
                    for (int x = 0; x < 10; ++x) st[LT::kCols + 10 * mb + x] = P[mb][x];
                bd2_ck_store<L::kN, L::kNP>(u == 0 ? ck_a : ck_b, threadIdx.x, st);
            }
            const float2 gc = *(const float2 *)(gg + 2 * u);                          // alpha, c
            const float2 rb = *(const float2 *)(rg + u * Stage<DK>::kRowFloats);      // beta, beta*v
            const float *ct = cg + u * Stage<DK>::kColFloats;
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < LT::kNVec; ++m) {
                float kk[4], k2[4], qq[4], mu[4];
                const int c0 = kLanesPerRow * 4 * m;
                vecf<4>::ld(ct + c0, kk);
                vecf<4>::ld(ct + DK + c0, k2);
                vecf<4>::ld(ct + 2 * DK + c0, qq);
                bd4_update(P[m], h + 4 * m, kk, k2, gc.x, gc.y, rb.x, rb.y);
                spd4_solve(P[m], h + 4 * m, mu);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = fmaf(mu[e], qq[e], acc);
            }
            part[u] = acc;
        }
        const float yv = row16_transpose_sum(part, g);
        const int tt = grp * kGroup + g;
        if (tt < left)
            yrow[(size_t)tt * ystride] = io<TOut>::from_f32(yv);
    }
}

// Same grid, staging and state I/O as bd2_fwd_kernel; P0 / PT are [B, H, dv, dk/4, 4, 4]
// (the upper triangle is read; PT is written in full, symmetric).
template <int DK, int C, typename TIn, typename TOut, bool CKPT = false>
__global__ __launch_bounds__(kThreads) void bd4_fwd_kernel(BdArgs a) {
    using LT = LaneTile<DK>;
    static_assert(LT::kVec == 4, "a lane's column vectors must be whole 4-blocks");
    constexpr int NB = LT::kNVec;                        // 4-blocks per lane
    extern __shared__ float lds[];
    float *buf0 = lds;
    float *buf1 = lds + C * Stage<DK>::kTokFloats;
    const int rb_per_head = a.dv / kRowsPerWG;
    int wg = blockIdx.x;
    if (a.xcd_remap) {
        const int per_xcd = a.nwg / 8;
        wg = (wg % 8) * per_xcd + wg / 8;
    }
    const int bh = wg / rb_per_head;
    const int row0 = (wg % rb_per_head) * kRowsPerWG;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane & (kLanesPerRow - 1);
    const int row_local = wave * kRowsPerWave + (lane >> 4);
    const int row = row0 + row_local;
    const float A = a.A[h], Ip = a.Ip[h];
    constexpr int kUp[10] = {0, 1, 2, 3, 5, 6, 7, 10, 11, 15};   // upper triangle in a row-major 4x4 block

    // state: h = P mu per entry, the upper triangle of P per 4-block
    float hv[4 * NB], P[NB][10];
    const size_t srow = ((size_t)bh * a.dv + row) * DK;      // entry (b, h, row, 0)
#pragma unroll
    for (int m = 0; m < NB; ++m) {
        const int col = LT::col(g, m, 0);                     // the block's first column
        if (a.mu0) {
            const float *pb = a.P0 + (srow + col) * 4;          // block (col / 4): 16 floats
            float full[16], mu[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) vecf<4>::ld(pb + 4 * q4, full + 4 * q4);
#pragma unroll
            for (int e = 0; e < 4; ++e) mu[e] = a.mu0[srow + col + e];
#pragma unroll
            for (int x = 0; x < 10; ++x) P[m][x] = full[kUp[x]];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // h = P mu with P symmetric from its upper triangle
                float acc = 0.f;
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) acc = fmaf(full[r < cc ? 4 * r + cc : 4 * cc + r], mu[cc], acc);
                hv[4 * m + r] = acc;
            }
        } else {
#pragma unroll
            for (int x = 0; x < 10; ++x) P[m][x] = (x == 0 || x == 4 || x == 7 || x == 9) ? Ip : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) hv[4 * m + e] = 0.f;
        }
    }

    const size_t seq = (size_t)b * a.T * a.H + h;
    const TIn *kseq = (const TIn *)a.k + seq * DK;
    const TIn *qseq = (const TIn *)a.q + seq * DK;
    const TIn *vseq = (const TIn *)a.v + seq * a.dv + row0;
    const TIn *bseq = (const TIn *)a.beta + seq * a.dv + row0;
    const TIn *dseq = (const TIn *)a.dt + seq;
    const size_t kq_tok = (size_t)a.H * DK, vb_tok = (size_t)a.H * a.dv;
    const size_t ystride = (size_t)a.H * a.dv;
    TOut *ybase = (TOut *)a.y + seq * a.dv + row;
    const size_t ck_stride = CKPT ? (size_t)rb_per_head * kThreads * BdLane<DK, 4>::kNP : 0;
    float *ckb = CKPT ? a.ck + ((size_t)bh * a.nsb * rb_per_head + wg % rb_per_head) *
                                   (kThreads * BdLane<DK, 4>::kNP)
                      : nullptr;
    // sub-block sb's checkpoint block, or the discard block past the sequence
    auto ck_at = [&](int sb) { return !CKPT ? nullptr : sb < a.nsb ? ckb + (size_t)sb * ck_stride : a.ck_sink; };
    const int nchunks = (a.T + C - 1) / C;
    Stager<DK, C, TIn, true> st;
    if (nchunks > 0) {
        st.load(kseq, qseq, vseq, bseq, dseq, a.T, a.H, a.dv, tid);
        st.commit(buf0, A, Ip, tid, false);
        __syncthreads();
    }
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C;
        const bool more = c + 1 < nchunks;
        if (more) {
            const size_t tn = (size_t)(t0 + C);
            st.load(kseq + tn * kq_tok, qseq + tn * kq_tok, vseq + tn * vb_tok, bseq + tn * vb_tok,
                    dseq + tn * a.H, a.T - (t0 + C), a.H, a.dv, tid);
        }
        bd4_chunk<DK, C, TOut, CKPT>((c & 1) ? buf1 : buf0, a.T - t0, hv, P, row_local, g,
                                     ybase + (size_t)t0 * ystride, ystride, ck_at(t0 / kSB), ck_at(t0 / kSB + 1));
        if (more) st.commit((c & 1) ? buf0 : buf1, A, Ip, tid, false);
        __syncthreads();
    }
    if (a.muT) {
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            const int col = LT::col(g, m, 0);
            float mu[4];
            if (a.T == 0 && a.mu0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) mu[e] = a.mu0[srow + col + e];   // copied through exactly
            } else {
                spd4_solve(P[m], hv + 4 * m, mu);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) a.muT[srow + col + e] = mu[e];
            const float *p = P[m];
            float *pb = a.PT + (srow + col) * 4;
            *(float4 *)pb = make_float4(p[0], p[1], p[2], p[3]);
            *(float4 *)(pb + 4) = make_float4(p[1], p[4], p[5], p[6]);
            *(float4 *)(pb + 8) = make_float4(p[2], p[5], p[7], p[8]);
            *(float4 *)(pb + 12) = make_float4(p[3], p[6], p[8], p[9]);
        }
    }
}

// ---------------------------------------------------------------------------
// block-diagonal precision, 4x4 blocks: backward
// ---------------------------------------------------------------------------
//
// The 2x2 backward's reverse walk with 4x4 blocks: per token and block the
// Cholesky factor of P_t serves both solves, mu = P^-1 h and w = P^-1 (gy_i q);
// S = sym(G_P) is kept as its upper triangle (10 floats), and the row sums
// weight S's off-diagonal entries twice in <S, P_prev>.  A lane state is 28
// floats at d = 128, so the walk replays quarters of 2 tokens from the
// checkpoint (20 replayed updates per 8 tokens) to hold two states, not four.

// Index of entry (i, j) of a symmetric 4x4 block in its upper-triangle storage.
__host__ __device__ constexpr int up4(int i, int j) {
    return i <= j ? (i * (7 - i)) / 2 + j : (j * (7 - j)) / 2 + i;
}

// The lane's start state: from (mu0, P0) when given (P0's upper triangle),
// else mu0 = 0 and P0 = I_prior Id.  srow: entry (b, h, row, 0).
template <int DK>
__device__ inline void bd4_start(const float *mu0, const float *P0, size_t srow, int g, float Ip, float *st) {
    using LT = LaneTile<DK>;
    constexpr int KC = LT::kCols;
#pragma unroll
    for (int m = 0; m < LT::kNVec; ++m) {
        float *p = st + KC + 10 * m, *hh = st + 4 * m;
        const int col = LT::col(g, m, 0);
        if (mu0) {
            const float *pb = P0 + (srow + col) * 4;
            float mu[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) mu[e] = mu0[srow + col + e];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = i; j < 4; ++j) p[up4(i, j)] = pb[4 * i + j];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) acc = fmaf(p[up4(i, j)], mu[j], acc);
                hh[i] = acc;
            }
        } else {
#pragma unroll
            for (int x = 0; x < 10; ++x) p[x] = (x == 0 || x == 4 || x == 7 || x == 9) ? Ip : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) hh[e] = 0.f;
        }
    }
}

// One token's update of the lane's 4-blocks (bd4_update, as the forward runs it).
template <int DK>
__device__ inline void bd4_update_lane(const float *ct, float alpha, float c, float beta, float bv, float *st) {
    using LT = LaneTile<DK>;
    constexpr int KC = LT::kCols;
#pragma unroll
    for (int m = 0; m < LT::kNVec; ++m) {
        float kk[4], k2[4];
        const int c0 = kLanesPerRow * 4 * m;
        vecf<4>::ld(ct + c0, kk);
        vecf<4>::ld(ct + DK + c0, k2);
        bd4_update(st + KC + 10 * m, st + 4 * m, kk, k2, alpha, c, beta, bv);
    }
}

// One token of the reverse walk for the lane's 4-blocks (St after the token,
// Sp before it); outputs as bd2_reverse_token.
template <int DK>
__device__ inline void bd4_reverse_token(const float *buf, int e, const float *St, const float *Sp, float *Gh,
                                         float *GS, int row_local, int g, int lane, float *red,
                                         float &cbv, float &cb, float &s1, float &s2) {
    using LT = LaneTile<DK>;
    using S = BwdStage<DK>;
    constexpr int KC = LT::kCols;
    const float alpha = buf[S::kGate + 2 * e];
    const float4 rw = *(const float4 *)(buf + S::kRows + e * S::kRowFloats + 4 * row_local);
    const float b2 = 2.f * rw.x, bv = rw.y, gy = rw.w;
    const float *ct = buf + e * S::kColFloats + LT::col(g, 0, 0);
    float dq[KC], dk[KC];
    cbv = 0.f; cb = 0.f; s1 = 0.f; s2 = 0.f;
#pragma unroll
    for (int m = 0; m < LT::kNVec; ++m) {
        float kk[4], qq[4];
        const int c0 = kLanesPerRow * 4 * m;
        vecf<4>::ld(ct + c0, kk);
        vecf<4>::ld(ct + 2 * DK + c0, qq);
        const float *p = St + KC + 10 * m, *pp = Sp + KC + 10 * m;
        const float *hh = St + 4 * m, *hp = Sp + 4 * m;
        float *gh = Gh + 4 * m, *gs = GS + 10 * m;
        const Chol4 f = spd4_factor(p);
        float mu[4], gq4[4], w[4], sk[4];
        spd4_apply(f, hh, mu);
#pragma unroll
        for (int i = 0; i < 4; ++i) gq4[i] = gy * qq[i];
        spd4_apply(f, gq4, w);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dq[4 * m + i] = gy * mu[i];
            gh[i] += w[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            gs[up4(i, i)] = fmaf(-w[i], mu[i], gs[up4(i, i)]);
#pragma unroll
            for (int j = i + 1; j < 4; ++j)
                gs[up4(i, j)] = fmaf(-0.5f, fmaf(w[i], mu[j], w[j] * mu[i]), gs[up4(i, j)]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float acc = gs[up4(i, 0)] * kk[0];
#pragma unroll
            for (int j = 1; j < 4; ++j) acc = fmaf(gs[up4(i, j)], kk[j], acc);
            sk[i] = acc;
            dk[4 * m + i] = fmaf(gh[i], bv, b2 * sk[i]);
            cbv = fmaf(gh[i], kk[i], cbv);
            cb = fmaf(sk[i], kk[i], cb);
            s1 = fmaf(gh[i], hp[i], s1);
            s2 += gs[up4(i, i)];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s1 = fmaf(gs[up4(i, i)], pp[up4(i, i)], s1);
#pragma unroll
            for (int j = i + 1; j < 4; ++j) s1 = fmaf(2.f * gs[up4(i, j)], pp[up4(i, j)], s1);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) gh[i] *= alpha;
#pragma unroll
        for (int x = 0; x < 10; ++x) gs[x] *= alpha;
    }
    bwd_scatter_qk<DK>(dq, dk, lane, g, red);
}

template <int DK, typename TIn, typename TG>
// Two workgroups per CU, as bd2_bwd_kernel (at d = 128 a few values spill).
__global__ __launch_bounds__(kThreads, 2) void bd4_bwd_kernel(BdBwdArgs a) {
    using LT = LaneTile<DK>;
    using S = BwdStage<DK>;
    using L = BdLane<DK, 4>;
    static_assert(LT::kVec == 4, "a lane's column vectors must be whole 4-blocks");
    constexpr int KC = LT::kCols, NB = KC / 4, N = L::kN;
    extern __shared__ float lds[];
    float *red = lds + S::kRed;
    float *rs = lds + S::kRs;

    const int rb_per_head = a.dv / kRowsPerWG;
    int wg = blockIdx.x;
    if (a.xcd_remap) {
        const int per_xcd = a.nwg / 8;
        wg = (wg % 8) * per_xcd + wg / 8;
    }
    const int bh = wg / rb_per_head;
    const int rb = wg % rb_per_head;
    const int row0 = rb * kRowsPerWG;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane & (kLanesPerRow - 1);
    const int row_local = wave * kRowsPerWave + (lane >> 4);
    const float A = a.A[h], Ip = a.Ip[h];
    const size_t srow = ((size_t)bh * a.dv + row0 + row_local) * DK;
    const size_t seq0 = (size_t)b * a.T * a.H + h;
    const size_t bth = (size_t)a.B * a.T * a.H;
    const size_t kq_tok = (size_t)a.H * DK, vb_tok = (size_t)a.H * a.dv;

    float Gh[KC], GS[10 * NB];
    // gPT's block at entry o, symmetrised into the upper triangle u
    auto load_gpt = [&](size_t o, float *u) {
        if (!a.gPT) {
#pragma unroll
            for (int x = 0; x < 10; ++x) u[x] = 0.f;
            return;
        }
        const float *gb = a.gPT + o * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = i; j < 4; ++j) u[up4(i, j)] = i == j ? gb[5 * i] : 0.5f * (gb[4 * i + j] + gb[4 * j + i]);
    };
    auto store_gp0 = [&](size_t o, const float *u) {
        float *gb = a.gP0 + o * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float row[4] = {u[up4(i, 0)], u[up4(i, 1)], u[up4(i, 2)], u[up4(i, 3)]};
            vecf<4>::st(gb + 4 * i, row);
        }
    };
    // the final state's adjoint from (gmuT, gPT), given the final state st
    auto final_adjoint = [&](const float *st) {
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            const size_t o = srow + LT::col(g, m, 0);
            const Chol4 f = spd4_factor(st + KC + 10 * m);
            float gm[4], muT[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) gm[e] = a.gmuT ? a.gmuT[o + e] : 0.f;
            spd4_apply(f, st + 4 * m, muT);
            spd4_apply(f, gm, Gh + 4 * m);
            float *gs = GS + 10 * m;
            const float *w = Gh + 4 * m;
            load_gpt(o, gs);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gs[up4(i, i)] = fmaf(-w[i], muT[i], gs[up4(i, i)]);
#pragma unroll
                for (int j = i + 1; j < 4; ++j)
                    gs[up4(i, j)] = fmaf(-0.5f, fmaf(w[i], muT[j], w[j] * muT[i]), gs[up4(i, j)]);
            }
        }
    };

    if (a.nsb == 0) {
        // T = 0: mu_T = mu_0 and P_T = P_0 are copied through, so are their gradients
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            const size_t o = srow + LT::col(g, m, 0);
            load_gpt(o, GS + 10 * m);
            if (a.gmu0)
#pragma unroll
                for (int e = 0; e < 4; ++e) a.gmu0[o + e] = a.gmuT ? a.gmuT[o + e] : 0.f;
            if (a.gP0) store_gp0(o, GS + 10 * m);
        }
    } else {
        const size_t ck_stride = (size_t)rb_per_head * kThreads * L::kNP;
        const float *ckb = a.ck + ((size_t)bh * a.nsb * rb_per_head + rb) * (kThreads * L::kNP);
        const TIn *kseq = (const TIn *)a.k + seq0 * DK;
        const TIn *qseq = (const TIn *)a.q + seq0 * DK;
        const TIn *vseq = (const TIn *)a.v + seq0 * a.dv + row0;
        const TIn *bseq = (const TIn *)a.beta + seq0 * a.dv + row0;
        const TG *gseq = (const TG *)a.gy + seq0 * a.dv + row0;
        const TIn *dseq = (const TIn *)a.dt + seq0;
        BwdStager<DK, TIn, TG> st;
        {
            const size_t tn = (size_t)(a.nsb - 1) * kSB;
            st.load(kseq + tn * kq_tok, qseq + tn * kq_tok, vseq + tn * vb_tok, bseq + tn * vb_tok,
                    gseq + tn * vb_tok, dseq + tn * a.H, a.T - (int)tn, a.H, a.dv, tid);
            st.commit(lds + ((a.nsb - 1) & 1) * S::kFloats, A, Ip, tid, false);
        }
        float ckS[N];
        bd2_ck_load<N, L::kNP>(ckb + (size_t)(a.nsb - 1) * ck_stride, tid, ckS);
        __syncthreads();

        for (int sb = a.nsb - 1; sb >= 0; --sb) {
            const float *cur = lds + (sb & 1) * S::kFloats;
            const int t0 = sb * kSB;
            // the checkpoint (loaded at the end of the previous sub-block) is
            // waited for before the next loads go out, not behind them
            regs_ready<N>(ckS);
            if (sb > 0) {
                const size_t tn = (size_t)(t0 - kSB);
                st.load(kseq + tn * kq_tok, qseq + tn * kq_tok, vseq + tn * vb_tok, bseq + tn * vb_tok,
                        gseq + tn * vb_tok, dseq + tn * a.H, a.T - (int)tn, a.H, a.dv, tid);
            }
            auto replay = [&](int e, float *x) {
                const float2 gc = *(const float2 *)(cur + S::kGate + 2 * e);
                const float2 rw = *(const float2 *)(cur + S::kRows + e * S::kRowFloats + 4 * row_local);
                bd4_update_lane<DK>(cur + e * S::kColFloats + LT::col(g, 0, 0), gc.x, gc.y, rw.x, rw.y, x);
            };
            float acc[16];      // this half's row partials: gbv, gb, da, dc of its 4 tokens
            // tokens 2qd and 2qd + 1, replayed from the checkpoint, walked in reverse
            auto quarter = [&](const int qd) {
                float mS[N], x0[N], x1[N];
#pragma unroll
                for (int i = 0; i < N; ++i) mS[i] = ckS[i];
                // ckS is dead after the last quarter's copy: the next checkpoint goes there
                if (qd == 0 && sb > 0) bd2_ck_load<N, L::kNP>(ckb + (size_t)(sb - 1) * ck_stride, tid, ckS);
                for (int e = 0; e < 2 * qd; ++e) replay(e, mS);
#pragma unroll
                for (int i = 0; i < N; ++i) x0[i] = mS[i];
                replay(2 * qd, x0);
#pragma unroll
                for (int i = 0; i < N; ++i) x1[i] = x0[i];
                replay(2 * qd + 1, x1);
                if (qd == 3 && sb == a.nsb - 1) final_adjoint(x1);   // tokens past T are neutral
                const int e1 = 2 * qd + 1, e0 = 2 * qd;
                __builtin_amdgcn_sched_barrier(0);
                bd4_reverse_token<DK>(cur, e1, x1, x0, Gh, GS, row_local, g, lane,
                                      red + (e1 * kWaves + wave) * 2 * DK,
                                      acc[e1 % 4], acc[e1 % 4 + 4], acc[e1 % 4 + 8], acc[e1 % 4 + 12]);
                __builtin_amdgcn_sched_barrier(0);
                bd4_reverse_token<DK>(cur, e0, x0, mS, Gh, GS, row_local, g, lane,
                                      red + (e0 * kWaves + wave) * 2 * DK,
                                      acc[e0 % 4], acc[e0 % 4 + 4], acc[e0 % 4 + 8], acc[e0 % 4 + 12]);
                __builtin_amdgcn_sched_barrier(0);
            };
            quarter(3);
            quarter(2);
            bwd_row_sums(acc, g, rs + 4 * 4 * kRowsPerWG + row_local);
            if (sb > 0) st.ready();    // half a sub-block after the loads, before any store
            quarter(1);
            quarter(0);
            bwd_row_sums(acc, g, rs + row_local);
            if (sb > 0) st.commit(lds + ((sb - 1) & 1) * S::kFloats, A, Ip, tid, false);
            __syncthreads();
            bd_bwd_epilogue<DK>(a, cur, red, rs, tid, t0, rb, bh, row0, seq0, bth);
            __syncthreads();
        }
        // the start state h_0 = P_0 mu_0: gmu0 = P_0 G_h, gP0 = S + sym(G_h mu0^T)
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            const size_t o = srow + LT::col(g, m, 0);
            float p0[10], m0[4] = {0.f, 0.f, 0.f, 0.f};
            float *gs = GS + 10 * m;
            const float *gh = Gh + 4 * m;
            if (a.mu0) {
                const float *pb = a.P0 + o * 4;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = i; j < 4; ++j) p0[up4(i, j)] = pb[4 * i + j];
#pragma unroll
                for (int e = 0; e < 4; ++e) m0[e] = a.mu0[o + e];
            } else {
#pragma unroll
                for (int x = 0; x < 10; ++x) p0[x] = (x == 0 || x == 4 || x == 7 || x == 9) ? Ip : 0.f;
            }
            if (a.gmu0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float acc = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc = fmaf(p0[up4(i, j)], gh[j], acc);
                    a.gmu0[o + i] = acc;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gs[up4(i, i)] = fmaf(gh[i], m0[i], gs[up4(i, i)]);
#pragma unroll
                for (int j = i + 1; j < 4; ++j)
                    gs[up4(i, j)] = fmaf(0.5f, fmaf(gh[i], m0[j], gh[j] * m0[i]), gs[up4(i, j)]);
            }
            if (a.gP0) store_gp0(o, gs);
        }
    }
    // this row block's sum of tr(gP0) (the default start P_0 = I_prior Id feeds gI_prior)
    float gsum = 0.f;
#pragma unroll
    for (int m = 0; m < NB; ++m) gsum += (GS[10 * m] + GS[10 * m + 4]) + (GS[10 * m + 7] + GS[10 * m + 9]);
    bd_bwd_trace_partial(a, gsum, rs, tid, (size_t)bh * rb_per_head + rb);
}

// Checkpoint pass of either block size: the forward's update without readout,
// staged like the forward (no q), storing the state before tokens 0, 8, 16, ...
template <int DK, int BS, typename TIn>
__global__ __launch_bounds__(kThreads) void bd_ckpt_kernel(BdBwdArgs a) {
    using LT = LaneTile<DK>;
    using L = BdLane<DK, BS>;
    using SG = Stage<DK>;
    constexpr int C = 16;
    extern __shared__ float lds[];
    const int rb_per_head = a.dv / kRowsPerWG;
    int wg = blockIdx.x;
    if (a.xcd_remap) {
        const int per_xcd = a.nwg / 8;
        wg = (wg % 8) * per_xcd + wg / 8;
    }
    const int bh = wg / rb_per_head, rb = wg % rb_per_head;
    const int row0 = rb * kRowsPerWG;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane & (kLanesPerRow - 1);
    const int row_local = wave * kRowsPerWave + (lane >> 4);
    const float A = a.A[h], Ip = a.Ip[h];
    float st[L::kN];
    if constexpr (BS == 2) bd2_start<DK>(a.mu0, a.P0, ((size_t)bh * a.dv + row0 + row_local) * DK, g, Ip, st);
    else bd4_start<DK>(a.mu0, a.P0, ((size_t)bh * a.dv + row0 + row_local) * DK, g, Ip, st);
    const size_t ck_stride = (size_t)rb_per_head * kThreads * L::kNP;
    float *ckb = a.ck + ((size_t)bh * a.nsb * rb_per_head + rb) * (kThreads * L::kNP);

    const size_t seq = (size_t)b * a.T * a.H + h;
    const TIn *kseq = (const TIn *)a.k + seq * DK;
    const TIn *vseq = (const TIn *)a.v + seq * a.dv + row0;
    const TIn *bseq = (const TIn *)a.beta + seq * a.dv + row0;
    const TIn *dseq = (const TIn *)a.dt + seq;
    const size_t kq_tok = (size_t)a.H * DK, vb_tok = (size_t)a.H * a.dv;
    const int nchunks = (a.T + C - 1) / C;
    Stager<DK, C, TIn, false> sg;
    sg.load(kseq, kseq, vseq, bseq, dseq, a.T, a.H, a.dv, tid);
    sg.commit(lds, A, Ip, tid, false);
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C;
        const bool more = c + 1 < nchunks;
        if (more) {
            const size_t tn = (size_t)(t0 + C);
            sg.load(kseq + tn * kq_tok, kseq + tn * kq_tok, vseq + tn * vb_tok, bseq + tn * vb_tok,
                    dseq + tn * a.H, a.T - (t0 + C), a.H, a.dv, tid);
        }
        const float *buf = lds + (c & 1) * C * SG::kTokFloats;
        const float *rows = buf + C * SG::kColFloats + 2 * row_local;
        const float *gates = buf + C * (SG::kColFloats + SG::kRowFloats);
#pragma unroll 2
        for (int u = 0; u < C; ++u) {
            if (u % kSB == 0 && (t0 + u) / kSB < a.nsb)
                bd2_ck_store<L::kN, L::kNP>(ckb + (size_t)((t0 + u) / kSB) * ck_stride, tid, st);
            const float2 gc = *(const float2 *)(gates + 2 * u);
            const float2 rw = *(const float2 *)(rows + u * SG::kRowFloats);
            if constexpr (BS == 2)
                bd2_update<DK>(buf + u * SG::kColFloats + LT::col(g, 0, 0), gc.x, gc.y, rw.x, rw.y, st);
            else
                bd4_update_lane<DK>(buf + u * SG::kColFloats + LT::col(g, 0, 0), gc.x, gc.y, rw.x, rw.y, st);
        }
        if (more) sg.commit(lds + ((c + 1) & 1) * C * SG::kTokFloats, A, Ip, tid, false);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// wide heads (d_k >= 512): one value row per wave
// ---------------------------------------------------------------------------
//
// For a head as wide as the model (the pages' recurrent-kernel measurement
// runs one head of width up to 2048, slides frame 22 / Fig. 7) a lane tile of
// one row and d_k/16 columns would not fit in registers.  Here each wave
// owns one value row and its 64 lanes split the columns (d_k/64 each, as
// 4-wide vectors spaced 256 apart, so a wave reads 1 KiB of contiguous LDS
// per vector); a workgroup of 4 waves owns 4 rows.  The per-column operands
// k, k^2, q of a chunk of kChunk tokens are staged once per workgroup as in
// the forward.  Each token's row sum is a whole-wave reduction (a DPP row sum,
// then the wave's 4 rows added with two permlane swaps: 8 VALU per token and
// lane, against 8 d_k/64 slots of updates).  Tokens are a rolled loop so that
// a lane holds one token's operands at a time.  The update is the forward's:
// 6 VALU + 1 v_rcp_f32 per entry.
template <int D> struct WideCfg {
    static constexpr int kCols = D / 64;                 // columns per lane
    static constexpr int kVecs = kCols / 4;              // 4-wide vectors per lane
    // tokens per staged chunk: 4 at 512 and 2 above, with k^2 staged up to
    // 1024 and computed in the lane at 2048, so that the double buffer takes
    // 49-66 KB (two or three workgroups per CU) and each chunk's global loads
    // have at least two tokens of compute to arrive
    static constexpr int kChunk = D == 512 ? 4 : 2;
    static constexpr bool kStageK2 = D < 2048;
    static constexpr int kRowsPerWave = D >= 2048 ? 1 : 2;   // rows per wave: a lane holds each one's entries of its columns
    static constexpr int kRows = 4 * kRowsPerWave;       // value rows per workgroup
    static constexpr int kColFloats = (kStageK2 ? 3 : 2) * D;   // k, (k^2), q per token
    static constexpr int kQ = (kStageK2 ? 2 : 1) * D;    // offset of q in a token
    static constexpr int kTokFloats = kColFloats + 2 * kRows + 2;
    static constexpr int kBufFloats = kChunk * kTokFloats;
    static_assert(kChunk >= 1, "at least one token per chunk");
    __device__ static inline int col(int lane, int m, int e) { return 256 * m + 4 * lane + e; }
};

template <int D, typename TIn>
struct WideStager {
    using W = WideCfg<D>;
    static constexpr int C = W::kChunk;
    static constexpr int kPer = packet<TIn>::kN;
    static constexpr int kColPkts = D / kPer;
    static constexpr int kHalf = C * kColPkts;
    static constexpr int kKQPer = (2 * kHalf + kThreads - 1) / kThreads;
    uint4 kq[kKQPer];
    uint32_t vv, bb, dtv;  // raw bits (io<TIn>::bits) until the commit
    // thread slots: (token, row) pairs of (v, beta) on wave 1, dt on wave 2
    __device__ static inline int vb_slot(int tid) { return (tid + kThreads - 64) % kThreads; }
    __device__ static inline int dt_slot(int tid) { return (tid + kThreads - 128) % kThreads; }

    __device__ inline void load(const TIn *kb, const TIn *qb, const TIn *vb, const TIn *bb_, const TIn *db,
                                int left, int H, int dv, int tid) {
#pragma unroll
        for (int u = 0; u < kKQPer; ++u) {
            const int p = tid + u * kThreads;
            if ((2 * kHalf) % kThreads == 0 || p < 2 * kHalf) {
                const bool isq = p >= kHalf;
                const int pp = isq ? p - kHalf : p;
                const int tt = pp / kColPkts;
                const size_t off = (size_t)tt * H * D + (pp % kColPkts) * kPer;
                kq[u] = make_uint4(0, 0, 0, 0);
                if (tt < left) kq[u] = *(const uint4 *)((isq ? qb : kb) + off);
            }
        }
        const int pv = vb_slot(tid);
        if (pv < C * W::kRows) {
            const int tt = pv / W::kRows, r = pv % W::kRows;
            vv = 0; bb = 0;
            if (tt < left) {
                const size_t off = (size_t)tt * H * dv + r;
                vv = io<TIn>::bits(vb[off]);
                bb = io<TIn>::bits(bb_[off]);
            }
        }
        const int pd = dt_slot(tid);
        if (pd < C) {
            dtv = 0;
            if (pd < left) dtv = io<TIn>::bits(db[(size_t)pd * H]);
        }
    }
    __device__ inline void commit(float *buf, float A, float Ip, int tid) const {
        float *rows = buf + C * W::kColFloats;
        float *gates = rows + C * 2 * W::kRows;
#pragma unroll
        for (int u = 0; u < kKQPer; ++u) {
            const int p = tid + u * kThreads;
            if ((2 * kHalf) % kThreads == 0 || p < 2 * kHalf) {
                const bool isq = p >= kHalf;
                const int pp = isq ? p - kHalf : p;
                const int tt = pp / kColPkts;
                const int off = (pp % kColPkts) * kPer;
                float x[kPer];
                packet<TIn>::widen(kq[u], x);
                float *dst = buf + tt * W::kColFloats + off;
#pragma unroll
                for (int e = 0; e < kPer; e += 4) {
                    if (!isq) {
                        *(float4 *)(dst + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
                        if (W::kStageK2)
                            *(float4 *)(dst + D + e) = make_float4(x[e] * x[e], x[e + 1] * x[e + 1],
                                                                   x[e + 2] * x[e + 2], x[e + 3] * x[e + 3]);
                    } else {
                        *(float4 *)(dst + W::kQ + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
                    }
                }
            }
        }
        const int pv = vb_slot(tid);
        if (pv < C * W::kRows) {
            const float b = io<TIn>::from_bits(bb), v = io<TIn>::from_bits(vv);
            *(float2 *)(rows + 2 * pv) = make_float2(b, b * v);
        }
        const int pd = dt_slot(tid);
        if (pd < C)
            *(float2 *)(gates + 2 * pd) = gate(A, io<TIn>::from_bits(dtv), Ip);
    }
};

// Sum of x over the four 16-lane rows of a wave (every lane receives it).
__device__ inline float sum_rows4(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, typename TIn, typename TOut>
__global__ __launch_bounds__(kThreads) void wide_fwd_kernel(FwdArgs a) {
    using W = WideCfg<D>;
    constexpr int C = W::kChunk, KC = W::kCols, R = W::kRowsPerWave;
    extern __shared__ float lds[];
    const int rb_per_head = a.dv / W::kRows;
    int wg = blockIdx.x;
    if (a.xcd_remap) {
        const int per_xcd = a.nwg / 8;
        wg = (wg % 8) * per_xcd + wg / 8;
    }
    const int bh = wg / rb_per_head;
    const int row0 = (wg % rb_per_head) * W::kRows;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int rw = wave * R;                          // the wave's first row in the workgroup
    const float A = a.A[h], Ip = a.Ip[h];

    // state of the wave's R rows: the lane's KC columns of each
    float M[R][KC], I[R][KC];
    const size_t srow = ((size_t)bh * a.dv + row0 + rw) * D;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < W::kVecs; ++m) {
            float mu[4], ii[4];
            if (a.mu0) {
                vecf<4>::ld(a.mu0 + srow + (size_t)r * D + W::col(lane, m, 0), mu);
                vecf<4>::ld(a.I0 + srow + (size_t)r * D + W::col(lane, m, 0), ii);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) { mu[e] = 0.f; ii[e] = Ip; }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) { I[r][4 * m + e] = ii[e]; M[r][4 * m + e] = ii[e] * mu[e]; }
        }

    const size_t seq = (size_t)b * a.T * a.H + h;
    const TIn *kseq = (const TIn *)a.k + seq * D;
    const TIn *qseq = (const TIn *)a.q + seq * D;
    const TIn *vseq = (const TIn *)a.v + seq * a.dv + row0;
    const TIn *bseq = (const TIn *)a.beta + seq * a.dv + row0;
    const TIn *dseq = (const TIn *)a.dt + seq;
    const size_t kq_tok = (size_t)a.H * D, vb_tok = (size_t)a.H * a.dv;
    const size_t ystride = (size_t)a.H * a.dv;
    TOut *ybase = (TOut *)a.y + seq * a.dv + row0 + rw;
    const int nchunks = (a.T + C - 1) / C;
    WideStager<D, TIn> st;
    if (nchunks > 0) {
        st.load(kseq, qseq, vseq, bseq, dseq, a.T, a.H, a.dv, tid);
        st.commit(lds, A, Ip, tid);
        __syncthreads();
    }
#pragma unroll 1
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C;
        const bool more = c + 1 < nchunks;
        if (more) {
            const size_t tn = (size_t)(t0 + C);
            st.load(kseq + tn * kq_tok, qseq + tn * kq_tok, vseq + tn * vb_tok, bseq + tn * vb_tok,
                    dseq + tn * a.H, a.T - (t0 + C), a.H, a.dv, tid);
        }
        const float *cur = lds + (c & 1) * W::kBufFloats;
        const float *rows = cur + C * W::kColFloats + 2 * rw;
        int goff = C * (W::kColFloats + 2 * W::kRows);
        asm volatile("" : "+v"(goff));
        const float *gates = cur + goff;
        // the chunk's 2-4 tokens unrolled: the next token's LDS reads are
        // issued under the current token's arithmetic
#pragma unroll
        for (int u = 0; u < C; ++u) {
            const float2 gc = *(const float2 *)(gates + 2 * u);
            float2 rb[R];
#pragma unroll
            for (int r = 0; r < R; ++r) rb[r] = *(const float2 *)(rows + u * 2 * W::kRows + 2 * r);
            const float *ct = cur + u * W::kColFloats + 4 * lane;
            float acc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
            for (int m = 0; m < W::kVecs; ++m) {
                float kk[4], k2[4], qq[4];
                vecf<4>::ld(ct + 256 * m, kk);
                if (W::kStageK2) vecf<4>::ld(ct + D + 256 * m, k2);
                vecf<4>::ld(ct + W::kQ + 256 * m, qq);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 4 * m + e;
                    if (!W::kStageK2) k2[e] = kk[e] * kk[e];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const float w = fmaf(rb[r].x, k2[e], gc.y);
                        I[r][s] = fmaf(gc.x, I[r][s], w);
                        M[r][s] = fmaf(gc.x, M[r][s], rb[r].y * kk[e]);
                        const float rc = __builtin_amdgcn_rcpf(I[r][s]);
                        acc[r] = fmaf(M[r][s] * rc, qq[e], acc[r]);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float yv = sum_rows4(row16_sum(acc[r]));
                if (lane == 0 && t0 + u < a.T)
                    ybase[(size_t)(t0 + u) * ystride + r] = io<TOut>::from_f32(yv);
            }
        }
        if (more) st.commit(lds + ((c + 1) & 1) * W::kBufFloats, A, Ip, tid);
        __syncthreads();
    }
    if (a.muT) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < W::kVecs; ++m) {
                float mu[4], ii[4];
                const size_t o = srow + (size_t)r * D + W::col(lane, m, 0);
                if (a.T == 0 && a.mu0) {
                    vecf<4>::ld(a.mu0 + o, mu);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) mu[e] = M[r][4 * m + e] / I[r][4 * m + e];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) ii[e] = I[r][4 * m + e];
                vecf<4>::st(a.muT + o, mu);
                vecf<4>::st(a.IT + o, ii);
            }
    }
}

// ---------------------------------------------------------------------------
// wide heads, row-parallel form (d_k >= 512 with a workspace)
// ---------------------------------------------------------------------------
//
// At d_k = d_v = 2048 one head's state is 32 MB, far more than a workgroup can
// stage per token, and the column-parallel layout above spends LDS reads and a
// whole-wave reduction on every token.  Here lanes run along value rows: a
// wave owns 64 rows of one head and KCL consecutive key columns of each (2 KCL
// VGPRs of state per lane).  The column operands k_j, k_j^2, q_j of a token are
// then the same for all 64 lanes, so they come in by scalar loads and feed the
// FMAs as SGPR operands: the token loop is the update's 6 VALU + 1 v_rcp_f32
// per entry with no LDS traffic and no cross-lane reduction, and each lane
// sums its own KCL columns of the readout.
//
// A workgroup is kWrNW such waves on the same 64 rows and kWrNW * KCL adjacent
// columns (a column slice).  The waves' partial readouts meet in LDS every
// 8 or 16 tokens and are added in wave order; the NQ slices of a row block
// leave their sums in a workspace, and a last pass adds them in slice order
// and rounds to the output type.  A first pass lays each token's columns out
// as records (k^2 in float32, the raw k and q words, the gate (alpha, c)), so
// the scalar operands need no ALU work beyond widening bf16 (two SALU bit
// operations per pair of columns) and a group of columns arrives with four
// scalar loads off one address.
//
// The loop-carried FMAs are written so that the new I and M land in the
// registers of the old ones (in_place_fma): left to itself the register
// allocator rotates the 2 KCL state registers through the temporaries and
// pays a copy per entry and token.

constexpr int kWrNW = 16;   // waves per workgroup (one column slice)
// tokens per LDS reduction block: 16 (128 KB) where the registers allow one
// workgroup per CU anyway, 8 (64 KB) at 16 columns per lane
template <int KCL> constexpr int wr_tok() { return KCL >= 32 ? 16 : 8; }

typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// A load the compiler may issue as a scalar (SMEM) load: the address is
// uniform over the wave and the memory is not written by the kernel.
template <typename T>
__device__ inline T scalar_load(const void *p) {
    return *(const __attribute__((address_space(4))) T *)p;
}

// x = s * x + w with x's register as the destination (v_fma_f32, s an SGPR)
__device__ inline void in_place_fma(float &x, float s, float w) {
    asm("v_fma_f32 %0, %1, %0, %2" : "+v"(x) : "s"(s), "v"(w));
}

// A group of a wave's columns for one token as the prep pass lays it out and
// as it sits in SGPRs: k^2 in float32, k and q as raw 32-bit words of the
// input type (16 bf16 columns or 8 float32 ones), the token's gate (alpha,
// c), padded to a multiple of 16 bytes.  One record per (token, group): the
// kernel reads each with four scalar loads off one address.
template <typename TIn> struct ColGroup;
template <> struct ColGroup<bf16_t> {
    static constexpr int kCols = 16, kWords = 36;
    f32x16 k2;
    u32x8 k, q;
    f32x2 g;
    __device__ static inline float widen(uint32_t w, int j) {
        return __uint_as_float(j & 1 ? w & 0xffff0000u : w << 16);
    }
    __device__ inline float kc(int j) const { return widen(k[j / 2], j); }
    __device__ inline float qc(int j) const { return widen(q[j / 2], j); }
    __device__ inline void load(const uint32_t *r) {
        k2 = scalar_load<f32x16>(r);
        k = scalar_load<u32x8>(r + 16);
        q = scalar_load<u32x8>(r + 24);
        g = scalar_load<f32x2>(r + 32);
    }
};
template <> struct ColGroup<float> {
    static constexpr int kCols = 8, kWords = 28;
    f32x8 k2;
    u32x8 k, q;
    f32x2 g;
    __device__ inline float kc(int j) const { return __uint_as_float(k[j]); }
    __device__ inline float qc(int j) const { return __uint_as_float(q[j]); }
    __device__ inline void load(const uint32_t *r) {
        k2 = scalar_load<f32x8>(r);
        k = scalar_load<u32x8>(r + 8);
        q = scalar_load<u32x8>(r + 16);
        g = scalar_load<f32x2>(r + 24);
    }
};

struct WideRowsArgs {
    const void *v, *beta;
    const uint32_t *rec;   // [B, T, H, D / kCols] column-group records
    const float *Ip, *mu0, *I0;
    float *muT, *IT;
    float *part;           // [nq, B, T, H, dv]: each column slice's readout
    int B, T, H, D, dv, nq, nwg, xcd_remap;
};

// One column-group record per thread: k^2, the raw k and q words, the gate.
// The records are built in LDS and leave as whole 16-byte columns of the
// workgroup's block (256 records, contiguous in the output): written record
// by record, each store instruction would cover 64 separate 16-byte pieces
// 144 bytes apart, and the partial lines cost about three times the bytes.
template <typename TIn>
__global__ __launch_bounds__(256) void wide_prep_kernel(const TIn *q, const TIn *k, const TIn *dt, const float *A,
                                                        const float *Ip, uint32_t *rec, size_t ntok, int H, int D) {
    using CG = ColGroup<TIn>;
    constexpr int G = CG::kCols, W = CG::kWords, W4 = W / 4;
    static_assert(W % 4 == 0, "records are whole 16-byte packets");
    constexpr int kWordsKQ = G * (int)sizeof(TIn) / 4;   // words of k (and of q) in a group
    __shared__ uint4 blk[256 * W4];
    const int per_tok = D / G;
    const size_t i0 = (size_t)blockIdx.x * 256;
    const size_t nrec = ntok * per_tok;
    const size_t i = i0 + threadIdx.x;
    if (i < nrec) {
        const size_t tok = i / per_tok;
        const int c = (int)(i % per_tok) * G;
        uint4 *r = blk + threadIdx.x * W4;
        const uint4 *kp = (const uint4 *)(k + tok * D + c), *qp = (const uint4 *)(q + tok * D + c);
#pragma unroll
        for (int p = 0; p < kWordsKQ / 4; ++p) {
            const uint4 kw = kp[p];
            float x[packet<TIn>::kN];
            packet<TIn>::widen(kw, x);
#pragma unroll
            for (int e = 0; e < packet<TIn>::kN; e += 4)
                r[(p * packet<TIn>::kN + e) / 4] = make_uint4(__float_as_uint(x[e] * x[e]), __float_as_uint(x[e + 1] * x[e + 1]),
                                                              __float_as_uint(x[e + 2] * x[e + 2]),
                                                              __float_as_uint(x[e + 3] * x[e + 3]));
            r[G / 4 + p] = kw;
            r[(G + kWordsKQ) / 4 + p] = qp[p];
        }
        const int h = (int)(tok % H);
        const float2 gt = gate(A[h], io<TIn>::to_f32(dt[tok]), Ip[h]);
        r[(G + 2 * kWordsKQ) / 4] = make_uint4(__float_as_uint(gt.x), __float_as_uint(gt.y), 0u, 0u);
    }
    __syncthreads();
    const size_t valid = (nrec - i0 < 256 ? nrec - i0 : 256) * W4;   // packets of this block's records
    uint4 *out = (uint4 *)rec + i0 * W4;
#pragma unroll
    for (int n = 0; n < W4; ++n) {
        const int pkt = threadIdx.x + 256 * n;
        if ((size_t)pkt < valid) out[pkt] = blk[pkt];
    }
}

template <int KCL, typename TIn>
__global__ __launch_bounds__(kWrNW * 64) void wide_rows_kernel(WideRowsArgs a) {
    using CG = ColGroup<TIn>;
    constexpr int NW = kWrNW, CB = wr_tok<KCL>(), G = CG::kCols, NG = KCL / G, W = CG::kWords;
    static_assert(KCL % G == 0, "columns per lane come in whole groups");
    extern __shared__ float red[];   // [2][CB][NW][64] partial readouts
    int wg = blockIdx.x;
    if (a.xcd_remap) {
        const int per_xcd = a.nwg / 8;
        wg = (wg % 8) * per_xcd + wg / 8;
    }
    // row block fastest, then column slice, then head: the row blocks of one
    // slice share its records through an XCD's L2
    const int rbs = a.dv / 64;
    const int rb = wg % rbs;
    const int qs = (wg / rbs) % a.nq;
    const int bh = wg / rbs / a.nq;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int D = a.D, T = a.T;
    const int row = rb * 64 + lane;
    const int col0 = (qs * NW + wave) * KCL;

    float M[KCL], I[KCL];
    const size_t srow = ((size_t)bh * a.dv + row) * D + col0;
    if (a.mu0) {
#pragma unroll
        for (int m = 0; m < KCL; m += 4) {
            float mu[4], ii[4];
            vecf<4>::ld(a.mu0 + srow + m, mu);
            vecf<4>::ld(a.I0 + srow + m, ii);
#pragma unroll
            for (int e = 0; e < 4; ++e) { I[m + e] = ii[e]; M[m + e] = ii[e] * mu[e]; }
        }
    } else {
        const float Ip = a.Ip[h];
#pragma unroll
        for (int s = 0; s < KCL; ++s) { I[s] = Ip; M[s] = 0.f; }
    }

    const size_t seq = (size_t)b * T * a.H + h;   // token index of (b, t = 0, h)
    const size_t H = (size_t)a.H;
    const uint32_t *rp = a.rec + (seq * (D / G) + col0 / G) * W;   // the wave's first record
    const size_t tstep = H * (D / G) * W;                          // words between tokens
    const TIn *vp = (const TIn *)a.v + seq * a.dv + row;
    const TIn *bp = (const TIn *)a.beta + seq * a.dv + row;
    const size_t rstep = H * a.dv;
    const size_t slice = (size_t)a.B * T * H * a.dv;
    float *part = a.part + (size_t)qs * slice + seq * a.dv + rb * 64;

    // the lane's (beta, v), one token ahead, as raw bits
    uint32_t bn = io<TIn>::bits(bp[0]), vn = io<TIn>::bits(vp[0]);
    // Records are software-pipelined: group (t, gi) is in SGPRs before it is
    // used, and the loads of the group after it are issued as soon as it has
    // arrived.  Scalar loads complete out of order, so every wait is a wait
    // for all of them; the empty asm makes the next loads' address depend on
    // the current group, which places that one wait before they are issued,
    // and the group's arithmetic then hides their latency.
    CG nx;
    nx.load(rp);
    const int nblk = (T + CB - 1) / CB;
#pragma unroll 1
    for (int blk = 0; blk < nblk; ++blk) {
        const int t0 = blk * CB;
        const int nt = T - t0 < CB ? T - t0 : CB;
        float *buf = red + (blk & 1) * (CB * NW * 64);
#pragma unroll 1
        for (int u = 0; u < nt; ++u) {
            const size_t t = (size_t)(t0 + u);
            const bool last = t0 + u + 1 >= T;
            const float bt = io<TIn>::from_bits(bn), bv = bt * io<TIn>::from_bits(vn);
            if (!last) {
                bn = io<TIn>::bits(bp[(t + 1) * rstep]);
                vn = io<TIn>::bits(vp[(t + 1) * rstep]);
            }
            float acc = 0.f;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const CG cur = nx;
                // the next record: (t, gi + 1), else (t + 1, 0); the last
                // token's last group reloads itself (an in-bounds address)
                size_t off = gi + 1 < NG ? t * tstep + (gi + 1) * W : (last ? t * tstep + gi * W : (t + 1) * tstep);
                const uint32_t w0 = cur.k[0];
                asm volatile("" : "+s"(off) : "s"(w0));
                nx.load(rp + off);
                __builtin_amdgcn_sched_barrier(0);   // issue them before this group's arithmetic
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    const int s = gi * G + j;
                    in_place_fma(I[s], cur.g.x, fmaf(bt, cur.k2[j], cur.g.y));
                    in_place_fma(M[s], cur.g.x, bv * cur.kc(j));
                    const float y = M[s] * __builtin_amdgcn_rcpf(I[s]);
                    acc = s == 0 ? y * cur.qc(j) : fmaf(y, cur.qc(j), acc);
                }
            }
            buf[(u * NW + wave) * 64 + lane] = acc;
        }
        // the slice's readout of these tokens: waves added in order (the
        // other buffer is written next, and the block after that only once
        // every wave has passed the next barrier, i.e. finished this sum)
        __syncthreads();
        if (tid < nt * 64) {
            const int u = tid >> 6, r = tid & 63;
            float s = buf[u * NW * 64 + r];
#pragma unroll
            for (int w = 1; w < NW; ++w) s += buf[(u * NW + w) * 64 + r];
            part[(size_t)(t0 + u) * rstep + r] = s;
        }
    }
    if (a.muT) {
#pragma unroll
        for (int m = 0; m < KCL; m += 4) {
            float mu[4], ii[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) { mu[e] = M[m + e] / I[m + e]; ii[e] = I[m + e]; }
            vecf<4>::st(a.muT + srow + m, mu);
            vecf<4>::st(a.IT + srow + m, ii);
        }
    }
}

// y = the column slices' readouts added in slice order, rounded to TOut
template <typename TOut>
__global__ __launch_bounds__(256) void wide_sum_kernel(const float *part, TOut *y, size_t n, int nq) {
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    // all slices' loads in flight before the in-order sum (nq <= 4; slices past
    // nq reload the last one and are not added)
    float4 x[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = *(const float4 *)(part + (size_t)(q < nq ? q : nq - 1) * n + i);
    float4 s = x[0];
#pragma unroll
    for (int q = 1; q < 4; ++q)
        if (q < nq) { s.x += x[q].x; s.y += x[q].y; s.z += x[q].z; s.w += x[q].w; }
    y[i] = io<TOut>::from_f32(s.x);
    y[i + 1] = io<TOut>::from_f32(s.y);
    y[i + 2] = io<TOut>::from_f32(s.z);
    y[i + 3] = io<TOut>::from_f32(s.w);
}

// ---------------------------------------------------------------------------
// frozen-importance forward (the Mamba2 limit) on the matrix cores
// ---------------------------------------------------------------------------
//
// With the importance held at I_prior (slides frame "The Mamba2 limit enables
// a gradual model upgrade", Secs. 2.3-2.4) the recurrence is
//     mu_t = alpha_t mu_{t-1} + w_t (x) k_t,   w_t = beta_t . v_t / I_prior,
//     y_t  = mu_t q_t,
// a scalar-decay linear attention whose chunked form is dense: per chunk of
// 64 tokens with Lam_t = sum_{r<=t} (-A dt_r),
//     Y     = diag(e^Lam) Q S^T + (L . Q K^T) W,   L_ts = e^(Lam_t - Lam_s) [s <= t]
//     S_end = e^Lam_end S + W^T diag(e^(Lam_end - Lam)) K.
// All four products run on v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32
// accumulation); the state S stays in fp32 accumulators for the whole sequence.
//
// One workgroup owns 64 value rows of one head (see frozen_fwd_kernel for the
// split of its 8 waves into staging and compute).
// MFMA fragments (16x16x32): A lane l = row l%16, k = 8(l/16)+j; B lane l =
// column l%16, k = 8(l/16)+j; D lane l = rows 4(l/16)+r of column l%16.  The
// state is kept as S^T tiles in D layout, which are fed back as A operands of
// S Q^T with the k index permuted (4 consecutive j from each of two tiles);
// the matching B operand reads Q with the same permutation.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

constexpr int kFzC = 64;       // tokens per chunk
constexpr int kFzRows = 64;    // value rows per workgroup

struct FrozenArgs {
    const bf16_t *q, *k, *v, *beta, *dt;      // beta NULL: v already holds beta . v
    const float *A, *Ip, *mu0;
    void *y;
    float *muT;
    int B, T, H, dv;
    int y_bf16;
};

template <int DK>
struct FzLds {
    // One staging buffer (bf16 unless noted); two are used alternately.  All
    // arrays are token-major, as the inputs are; the operands that need the
    // token index along k (K^T, W^T) are read with gfx950's transposing LDS
    // read.  Q and K rows are padded by 8 elements (16 bytes) so that the 16
    // rows a fragment read touches fall in distinct LDS banks.  K is also
    // swizzled: the 16-byte column block cb of row r sits at block
    // cb ^ ((r / 8) % 8), which keeps the stagers' row writes (8 tokens apart)
    // in distinct banks too.  W rows are 80 elements apart (40 banks), so the
    // 8 token rows of a half-wave's transposing read hit distinct banks.
    static constexpr int kQS = DK + 8;                   // row stride of Q and K
    static constexpr int kWS = kFzRows + 16;             // row stride of W and diag(d) W
    static constexpr int kQ = 0;                         // Q  [C][DK]
    static constexpr int kK = kQ + kFzC * kQS;           // K  [C][DK]
    static constexpr int kW = kK + kFzC * kQS;           // W  [C][64]
    static constexpr int kWd = kW + kFzC * kWS;          // diag(d) W [C][64]
    static constexpr int kP = kWd + kFzC * kWS;          // P^T tiles [10][64 lanes][4], D-fragment order
    static constexpr int kBufHalves = kP + 10 * 256;
    static constexpr int kLamBytes = kFzC * 4;           // Lam [C] float, after the halves
    static constexpr int kBufBytes = kBufHalves * 2 + kLamBytes;
    // Two y tiles (chunk c in tile c&1), [C tokens][64 rows] in the output
    // type, rows 16 bytes longer than the data (144 or 272 bytes) so that the
    // 16 tokens of a compute wave's fragment write fall in distinct banks.
    static constexpr int kY = 2 * kBufBytes;
    static constexpr int kYTile = kFzC * (kFzRows * 4 + 16);
    // the W role's per-wave copy of the chunk's state weights [wave][64 tokens]
    static constexpr int kDl = kY + 2 * kYTile;
    static constexpr int kTotal = kDl + 4 * kFzC * 4;
};

// Dword i of a 16-byte packet, and the bf16 in its low / high half as float.
// (Indexing a register packet through a pointer would push it to scratch.)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ inline uint32_t u4get(const u32x4 &p, int i) { return p[i]; }

// Value of x in lane `src` (wave-uniform source lane).
__device__ inline float wave_read(float x, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), src));
}
// x of the lane CTRL's row shift names, or 0 where that lane is outside the row.
template <int CTRL>
__device__ inline float dpp_or_zero(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Inclusive prefix sum over the 64 lanes of a wave (all lanes active):
// Hillis-Steele within each 16-lane row (row_shr 1, 2, 4, 8), then each row
// adds the totals of the rows before it, read from lanes 15, 31, 47.
__device__ inline float wave_incl_scan(float x, int lane) {
    x += dpp_or_zero<0x111>(x);
    x += dpp_or_zero<0x112>(x);
    x += dpp_or_zero<0x114>(x);
    x += dpp_or_zero<0x118>(x);
    const float r0 = wave_read(x, 15), r1 = wave_read(x, 31), r2 = wave_read(x, 47);
    const int row = lane >> 4;
    const float before = row == 0 ? 0.f : row == 1 ? r0 : row == 2 ? r0 + r1 : (r0 + r1) + r2;
    return x + before;
}
__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Two floats to packed bf16 (round to nearest even) in one v_cvt_pk_bf16_f32;
// converting them one at a time and merging the halves takes four instructions.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2_t));
}
__device__ inline bf16x4_t cvt4_bf16(f32x4 x) { return __builtin_convertvector(x, bf16x4_t); }

__device__ inline bf16x8_t lds_b128(const bf16_t *p) { return *(const bf16x8_t *)p; }
__device__ inline bf16x4_t lds_b64(const bf16_t *p) { return *(const bf16x4_t *)p; }
__device__ inline bf16x8_t cat8(bf16x4_t x, bf16x4_t y) {
    return bf16x8_t{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}
// Four consecutive rows of one column through gfx950's transposing LDS read
// (ds_read_b64_tr_b16): lane m of each 16-lane group supplies the address of
// X[r + m / 4][c0 + 4 (m % 4)] (8 bytes) and receives X[r + e][c0 + m],
// e = 0..3, where r may differ between the four groups.  The pointer is the
// lane's own 8-byte source.
__device__ inline bf16x4_t lds_tr4(const bf16_t *src) {
    typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
    return __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)src));
}
// index of the lower-triangle score tile (s block sb <= query block tb)
__device__ constexpr int tri(int sb, int tb) { return tb * (tb + 1) / 2 + sb; }

// Score tiles of compute wave CW (s block, t block) as compile-time lists, so
// that the wave loads each distinct Q and K fragment once per k step: waves 0
// and 1 take three tiles, 2 and 3 two (4, 4, 3, 3 fragment reads per step).
// The tiles go to LDS as the decay-masked P^T = G^T e^(Lam_t - Lam_s) / I_prior
// (s <= t) in bf16, D-fragment order; the 1 / I_prior of w = beta v / I_prior
// is applied here (as -ln I_prior in the exponent) rather than to every
// element of W.
template <int DK, int CW>
__device__ inline void fz_scores(const bf16_t *hb, const float *lam, bf16_t *pw, int lane, float ln_inv_ip) {
    using L = FzLds<DK>;
    // 4, 3, 2, 1 tiles: waves 0 and 1 share their SIMDs with the K role,
    // whose phase A work (the y copy) is light, waves 2 and 3 with the W role's
    // commit; Q and K fragments read per k step: 4, 4, 3, 2
    constexpr int NT = 4 - CW;
    constexpr int kSb[4][4] = {{0, 1, 0, 1}, {0, 0, 1, 0}, {2, 2, 0, 0}, {3, 0, 0, 0}};
    constexpr int kTb[4][4] = {{2, 2, 3, 3}, {0, 1, 1, 0}, {2, 3, 0, 0}, {3, 0, 0, 0}};
    const int lr = lane & 15, lg = lane >> 4;
    f32x4 g[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) g[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) {
        bf16x8_t qf[4], kf[4];
#pragma unroll
        for (int bl = 0; bl < 4; ++bl) {
            bool uq = false, uk = false;
#pragma unroll
            for (int n = 0; n < NT; ++n) { uq |= kTb[CW][n] == bl; uk |= kSb[CW][n] == bl; }
            if (uq) qf[bl] = lds_b128(hb + L::kQ + (16 * bl + lr) * L::kQS + 32 * kk + 8 * lg);
            const int kr = 16 * bl + lr;
            if (uk) kf[bl] = lds_b128(hb + L::kK + kr * L::kQS + 8 * ((4 * kk + lg) ^ ((kr >> 3) & 7)));
        }
#pragma unroll
        for (int n = 0; n < NT; ++n)
            g[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kSb[CW][n]], qf[kTb[CW][n]], g[n], 0, 0, 0);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int sb = kSb[CW][n], tb = kTb[CW][n];
        const float lt = lam[16 * tb + lr] + ln_inv_ip;
        const f32x4 ls = *(const f32x4 *)(lam + 16 * sb + 4 * lg);
        f32x4 pt;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool keep = sb < tb || 4 * lg + r <= lr;
            pt[r] = keep ? g[n][r] * __expf(lt - ls[r]) : 0.f;
        }
        *(bf16x4_t *)(pw + 256 * tri(sb, tb)) = cvt4_bf16(pt);
    }
}

// Warp-specialised: waves 0-3 compute chunk c while waves 4-7 widen and
// stage chunk c+1 into the other LDS buffer and load chunk c+2 from HBM; two
// barriers per chunk.  The compute waves first form the 10 lower-triangle
// score tiles of the chunk between them and share them through LDS; then
// compute wave w, which owns value rows [16w, 16w+16) of the workgroup, forms
// Y for its rows and its part of the state.
template <int DK>
__global__ __launch_bounds__(512) void frozen_fwd_kernel(FrozenArgs a) {
    using L = FzLds<DK>;
    extern __shared__ float lds_f[];
    char *lds = (char *)lds_f;
    const int rb_per_head = a.dv / kFzRows;
    // consecutive workgroup ids go round-robin over the 8 XCDs; remap so that
    // the row blocks of one head, which read the same q and k, share an XCD's L2
    int wg = blockIdx.x;
    if (gridDim.x % 8 == 0) wg = (wg % 8) * (gridDim.x / 8) + wg / 8;
    const int bh = wg / rb_per_head;
    const int ib0 = (wg % rb_per_head) * kFzRows;      // first value row of the workgroup
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const bool stager = wv >= 4;
    const int w = wv & 3;
    const int lr = lane & 15, lg = lane >> 4;                 // fragment row/col and lane group
    const float Ah = a.A[h], inv_ip = 1.f / a.Ip[h], ln_inv_ip = -__logf(a.Ip[h]);
    const size_t seq = (size_t)b * a.T * a.H + h;            // [B, T, H] row of (b, 0, h)
    const int nchunks = (a.T + kFzC - 1) / kFzC;
    const int yesz = a.y_bf16 ? 2 : 4, yrow = 64 * yesz + 16;  // y element and LDS row bytes

    // ---- staging waves (threads 256..511, index u = tid - 256).  Roles:
    //   u in [0, DK):        one 8x8 block of K (tokens 8 (u % 8).., columns
    //                        8 (u / 8)..), written as K rows; and 8 packets of
    //                        Q (packet e DK + u in row-major order: consecutive
    //                        threads cover a token row)
    //   u in [DK, DK+128):   x = u - DK; two whole waves.  Each thread stages one
    //                        4-token x 8-row block of beta . v (tokens 4 (x/8)..,
    //                        rows 8 (x%8)..), written as W = beta . v and as
    //                        diag(d) W / I_prior rows; both waves scan the gate
    //                        (one token per lane) and the first writes Lam
    // The block assignments put the 16 lanes of one LDS write pass on rows or
    // tokens that fall in distinct banks.
    //   u >= DK+128:         idle (d_k = 64)
    // Loads read a valid row (clamped to T-1); past the end of the sequence
    // q = k = 0, dt = 0 and diag(d) W = 0 are staged (no effect on y or the
    // state; W keeps the last token's values, which meet only masked scores).
    const int u = tid - 256;
    constexpr int kQPk = DK / 8;            // 16-byte packets per Q row
    // 16-byte packets of this thread's role: the K role stages one chunk
    // from pr; the W role alternates between pr and pr2, two chunks ahead
    // dt stays in its bf16 bits until the commit: widening it at the load
    // would make the wave wait for the load there
    u32x4 pr[16], pr2[16];
    uint32_t pdt = 0, pdt2 = 0;
    // Token t of a [B, T, H, n] tensor starts at element (seq + t H) n; tokens
    // past the end are clamped to T-1.  Every load takes the same branch-free
    // address form: per-load branches would split the loads into blocks whose
    // register reuse makes the wave wait for earlier loads.
    // One lambda per role and no role test inside: each role's loop then has
    // straight-line loads, which the compiler counts, so a commit waits only
    // for the packets it uses.
    auto row = [&](int t) { return seq + (size_t)min(t, a.T - 1) * a.H; };
    auto load_k = [&](int t0) __attribute__((always_inline)) {
        const int tok0 = 8 * (u % 8), col = 8 * (u / 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) pr[e] = *(const u32x4 *)(a.k + row(t0 + tok0 + e) * DK + col);
        const int tq0 = u / kQPk, qcol = 8 * (u % kQPk);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            pr[8 + e] = *(const u32x4 *)(a.q + row(t0 + e * (DK / kQPk) + tq0) * DK + qcol);
    };
    // W role: x = u - DK; with d_k = 64 the role's third wave (x >= 128) loads
    // the first wave's packets and stores nothing
    const int wx = u - DK, wxl = wx & 127;
    auto load_w = [&](int t0, u32x4 *p, uint32_t &d) __attribute__((always_inline)) {
        const int tok0 = 4 * (wxl / 8), i0 = ib0 + 8 * (wxl % 8);
        const bf16_t *bsrc = a.beta ? a.beta : a.v;    // no beta: replaced by 1.0 at the commit
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t o = row(t0 + tok0 + e) * a.dv + i0;
            p[e] = *(const u32x4 *)(a.v + o);
            p[4 + e] = *(const u32x4 *)(bsrc + o);
        }
        d = __builtin_bit_cast(uint16_t, a.dt[row(t0 + lane)]);
    };
    auto commit_k = [&](char *buf, int t0) __attribute__((always_inline)) {
        bf16_t *hb = (bf16_t *)buf;
        const u32x4 z = u32x4{0u, 0u, 0u, 0u};
        const int tok0 = 8 * (u % 8);
        const int pcol = 8 * ((u / 8) ^ (u % 8));     // swizzled column block (rows tok0.. share r / 8)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            *(u32x4 *)(hb + L::kK + (tok0 + e) * L::kQS + pcol) = (t0 + tok0 + e < a.T) ? pr[e] : z;
        const int tq0 = u / kQPk, qcol = 8 * (u % kQPk);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int tq = e * (DK / kQPk) + tq0;
            *(u32x4 *)(hb + L::kQ + tq * L::kQS + qcol) = (t0 + tq < a.T) ? pr[8 + e] : z;
        }
    };
    auto commit_w = [&](char *buf, int t0, const u32x4 *p, uint32_t d) __attribute__((always_inline)) {
        bf16_t *hb = (bf16_t *)buf;
        float *lam = (float *)(buf + L::kBufHalves * 2);
        // gate: Lam = inclusive prefix sum of -A dt over the chunk, lane = token
        const float lam_l = wave_incl_scan((t0 + lane < a.T) ? -Ah * __uint_as_float(d << 16) : 0.f, lane);
        if (wx < 64) lam[lane] = lam_l;
        // e^(Lam_end - Lam_s) / I_prior: W is staged as beta . v, its 1 / I_prior
        // applied here for diag(d) W and in the score tiles for the readout.
        // Past the end of the sequence the weight is 0, so diag(d) W is 0
        // there; W itself keeps the (finite) values of the clamped last token,
        // which only meet score entries of token pairs s > t, masked to 0.
        const float dl = (t0 + lane < a.T) ? __expf(wave_read(lam_l, 63) - lam_l) * inv_ip : 0.f;
        const int tok0 = 4 * (wxl / 8), il0 = 8 * (wxl % 8);
        // the thread's four tokens' weights through the wave's own LDS slot
        // (one write and one 16-byte read instead of four lane shuffles)
        float *dls = (float *)(lds + L::kDl) + kFzC * (wx >> 6);
        dls[lane] = dl;
        const f32x4 d4 = *(const f32x4 *)(dls + tok0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float de = d4[e];
            uint32_t ww[4], wd[4];
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const uint32_t vw = u4get(p[e], pp);
                const uint32_t bw = a.beta ? u4get(p[4 + e], pp) : 0x3f803f80u;
                const float w0 = bf_lo(bw) * bf_lo(vw), w1 = bf_hi(bw) * bf_hi(vw);
                ww[pp] = pack_bf16(w0, w1);
                wd[pp] = pack_bf16(w0 * de, w1 * de);
            }
            if (wx < 128) {
                *(u32x4 *)(hb + L::kW + (tok0 + e) * L::kWS + il0) = u32x4{ww[0], ww[1], ww[2], ww[3]};
                *(u32x4 *)(hb + L::kWd + (tok0 + e) * L::kWS + il0) = u32x4{wd[0], wd[1], wd[2], wd[3]};
            }
        }
    };

    // Two phases per chunk, each closed by a barrier.  Phase A: the compute
    // waves form the chunk's 10 decay-masked score tiles, 1-4 per wave, and
    // share them through LDS; they also update the state, keeping the
    // previous one in bf16 for phase B.  Phase B: the compute waves form Y.
    // The stagers fill buffer (c+1)&1 (not read during chunk c) with chunk
    // c+1: the W role in phase A, the K role in phase B, so that each phase
    // carries about half of the chunk's LDS traffic (phase A's score and K^T
    // reads are the larger share; the K and Q writes are twice the W ones).
    // The roles run separate loops with the same barriers, so that no role's
    // registers stay reserved in another's code.  The K role copies y of
    // chunk c-1 out in phase A, then stages c+1 and loads c+2 in phase B
    // (loading c+2 in phase A instead, from a second register set, measured
    // no faster).  The W role loads chunk c+3 in phase B, alternating between
    // two register sets.  (Spreading both roles' work over all four staging
    // waves was slower: the compute waves are the critical path, and two of
    // them then share a SIMD with more staging.)
    auto buf_of = [&](int c) { return lds + (c & 1) * L::kBufBytes; };
    // The W role's packets of one register set, marked used before the other
    // set's loads go out, so that the wait for them (loads two phases old)
    // lands here and a commit never waits for loads issued a phase earlier.
    auto w_ready = [&](const u32x4 *p, uint32_t d) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) asm volatile("" ::"v"(p[e].x), "v"(p[e].y), "v"(p[e].z), "v"(p[e].w));
        asm volatile("" ::"v"(d));
    };
    // Every load batch is issued, for chunk min(c, nchunks - 1) (the surplus
    // ones near the end reload the last chunk and are never committed): a
    // batch under a branch is one the compiler cannot count, and it then waits
    // for all outstanding loads at the next commit.
    auto clampc = [&](int c) { return min(c, nchunks - 1) * kFzC; };
    if (stager && u < DK) {
        // y of chunk c (complete after chunk c's phase B) from its LDS tile to
        // HBM in 16-byte packets, whole output rows per group of threads
        auto write_y = [&](int c) __attribute__((always_inline)) {
            const int t0 = c * kFzC, ppr = 64 * yesz / 16;           // packets per token row
            const char *yt = lds + L::kY + (c & 1) * L::kYTile;
            for (int p = u; p < kFzC * ppr; p += DK) {
                const int t = p / ppr, col = 16 * (p % ppr);
                if (t0 + t < a.T)
                    *(u32x4 *)((char *)a.y + ((seq + (size_t)(t0 + t) * a.H) * a.dv + ib0) * yesz + col) =
                        *(const u32x4 *)(yt + t * yrow + col);
            }
        };
        if (nchunks > 0) {
            load_k(0);
            commit_k(lds, 0);
            load_k(clampc(1));
        }
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            // phase A: y of chunk c-1 out (its tile is next written in phase B of c+1)
            if (c > 0) write_y(c - 1);
            __syncthreads();
            // phase B: chunk c+1 into the other buffer, whose last reads were in chunk c-1
            if (c + 1 < nchunks) commit_k(buf_of(c + 1), (c + 1) * kFzC);
            load_k(clampc(c + 2));
            __syncthreads();
        }
        if (nchunks > 0) write_y(nchunks - 1);
        return;
    }
    if (stager) {
        if (nchunks > 0) {
            load_w(0, pr, pdt);
            commit_w(lds, 0, pr, pdt);
            load_w(clampc(1), pr2, pdt2);
            w_ready(pr2, pdt2);    // as in the loop: the loop head then never waits for pr
            load_w(clampc(2), pr, pdt);
        }
        __syncthreads();
        for (int c = 0; c < nchunks; c += 2) {
            if (c + 1 < nchunks) commit_w(buf_of(c + 1), (c + 1) * kFzC, pr2, pdt2);
            __syncthreads();
            w_ready(pr, pdt);
            load_w(clampc(c + 3), pr2, pdt2);
            __syncthreads();
            if (c + 1 >= nchunks) break;
            if (c + 2 < nchunks) commit_w(buf_of(c + 2), (c + 2) * kFzC, pr, pdt);
            __syncthreads();
            w_ready(pr2, pdt2);
            load_w(clampc(c + 4), pr, pdt);
            __syncthreads();
        }
        return;
    }

    // ---- compute waves: state S^T tiles (jb, rows of wave w); lane holds
    // S^T[16 jb + 4 lg + r][16 w + lr] = S[i][j]
    f32x4 St[DK / 16];
    const int irow = ib0 + 16 * w + lr;
    const size_t srow = ((size_t)bh * a.dv + irow) * DK;
    if (a.mu0) {
#pragma unroll
        for (int jb = 0; jb < DK / 16; ++jb) St[jb] = *(const f32x4 *)(a.mu0 + srow + 16 * jb + 4 * lg);
    } else {
#pragma unroll
        for (int jb = 0; jb < DK / 16; ++jb) St[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
        bf16x8_t sa[DK / 32];
        char *bufw = lds + (c & 1) * L::kBufBytes;
        const char *buf = bufw;
        const bf16_t *hb = (const bf16_t *)buf;
        const float *lam = (const float *)(buf + L::kBufHalves * 2);
        {
            // (a) scores G^T[s][t] = k_s . q_t of this wave's tiles, decay-masked, to LDS
            bf16_t *pw_ = (bf16_t *)bufw + L::kP + 4 * lane;
            switch (w) {
            case 0: fz_scores<DK, 0>(hb, lam, pw_, lane, ln_inv_ip); break;
            case 1: fz_scores<DK, 1>(hb, lam, pw_, lane, ln_inv_ip); break;
            case 2: fz_scores<DK, 2>(hb, lam, pw_, lane, ln_inv_ip); break;
            default: fz_scores<DK, 3>(hb, lam, pw_, lane, ln_inv_ip); break;
            }
            // the state before this chunk, as the bf16 A operand of S Q^T in phase B
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) sa[kk] = cat8(cvt4_bf16(St[2 * kk]), cvt4_bf16(St[2 * kk + 1]));
            // (e) state: S^T = e^Lam_end S^T + K^T diag(d) W
            const float e_end = __expf(lam[kFzC - 1]);
            // Operands with the token index along k, read transposed from the
            // token-major arrays: lane (lg, lr) supplies row 8 lg + lr / 4 (+4)
            // of its 32-token slice and columns 4 (lr % 4).. of its 16-column
            // block, and receives 8 consecutive tokens of one column.
            const int trow = 8 * lg + (lr >> 2), tcol = 4 * (lr & 3);
            bf16x8_t wd[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16_t *p = hb + L::kWd + (32 * ks + trow) * L::kWS + 16 * w + tcol;
                wd[ks] = cat8(lds_tr4(p), lds_tr4(p + 4 * L::kWS));
            }
            // k step outer: the DK/16 key blocks' products are independent, so
            // that many are in flight between the two dependent steps
#pragma unroll
            for (int jb = 0; jb < DK / 16; ++jb) St[jb] = St[jb] * e_end;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int jb = 0; jb < DK / 16; ++jb) {
                    // K^T fragment from the swizzled K rows (the 8 rows share r / 8)
                    const int r = 32 * ks + trow, c = 16 * jb + tcol;
                    const bf16_t *p = hb + L::kK + r * L::kQS + 8 * ((c >> 3) ^ ((r >> 3) & 7)) + (c & 7);
                    St[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cat8(lds_tr4(p), lds_tr4(p + 4 * L::kQS)), wd[ks],
                                                                    St[jb], 0, 0, 0);
                }
        }
        __syncthreads();
        {
            float lam_t[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) lam_t[tb] = lam[16 * tb + lr];
            const bf16_t *pr_t = hb + L::kP + 4 * lane;   // this lane's fragment of each P^T tile
            auto ptile = [&](int i) __attribute__((always_inline)) { return lds_b64(pr_t + 256 * i); };

            // (c) Y^T for value rows of wave w: intra-chunk W^T P^T + inter-chunk S Q^T e^Lam_t.
            // The k index (token s) of the intra product follows the P^T
            // fragments: slots 0-3 = s 4lg..4lg+3 of s block 2ks, slots 4-7 of block 2ks+1.
            // W^T fragments, read transposed from the token-major W: lane (lg, lr)
            // supplies token row 4 lg + lr / 4 (and 16 more) and value rows
            // 16 w + 4 (lr % 4).., and receives tokens 4 lg.. of value row 16 w + lr
            const bf16_t *wtr = hb + L::kW + (4 * lg + (lr >> 2)) * L::kWS + 16 * w + 4 * (lr & 3);
            const bf16x4_t zero4 = {(bf16_t)0.f, (bf16_t)0.f, (bf16_t)0.f, (bf16_t)0.f};
            // The two W^T fragments serve every query block; the four blocks'
            // inter-chunk chains run interleaved (k step outer), so that four
            // independent products are in flight instead of one chain of four.
            bf16x8_t av[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                av[ks] = cat8(lds_tr4(wtr + 32 * ks * L::kWS), lds_tr4(wtr + (32 * ks + 16) * L::kWS));
            f32x4 yi[4], ye[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                yi[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
                ye[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks <= tb / 2; ++ks) {
                    const bf16x8_t bv = cat8(ptile(tri(2 * ks, tb)), 2 * ks + 1 <= tb ? ptile(tri(2 * ks + 1 <= tb ? 2 * ks + 1 : 0, tb)) : zero4);
                    yi[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[ks], bv, yi[tb], 0, 0, 0);
                }
            }
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk)
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const bf16_t *qrow = hb + L::kQ + (16 * tb + lr) * L::kQS + 32 * kk + 4 * lg;
                    ye[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sa[kk], cat8(lds_b64(qrow), lds_b64(qrow + 16)),
                                                                    ye[tb], 0, 0, 0);
                }
            // y of the wave's rows into the chunk's LDS tile; the K-role stagers
            // write it out during the next chunk's phase A as whole rows (a
            // fragment store scatters 8 or 16 bytes per lane over 16 token rows)
            char *yt = lds + L::kY + (c & 1) * L::kYTile + (4 * lg + 16 * w) * yesz;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int t = 16 * tb + lr;
                const float et = __expf(lam_t[tb]);
                const f32x4 o = {fmaf(et, ye[tb][0], yi[tb][0]), fmaf(et, ye[tb][1], yi[tb][1]),
                                 fmaf(et, ye[tb][2], yi[tb][2]), fmaf(et, ye[tb][3], yi[tb][3])};
                if (a.y_bf16) *(bf16x4_t *)(yt + t * yrow) = cvt4_bf16(o);
                else *(f32x4 *)(yt + t * yrow) = o;
            }
        }
        __syncthreads();
    }
    if (a.muT) {
#pragma unroll
        for (int jb = 0; jb < DK / 16; ++jb)
            *(f32x4 *)(a.muT + srow + 16 * jb + 4 * lg) = St[jb];
    }
}

// ---------------------------------------------------------------------------
// decode step
// ---------------------------------------------------------------------------

struct StepArgs {
    const void *q, *k, *v, *beta, *dt;
    const float *A, *Ip;
    float *mu, *I;
    void *y;
    int B, H, dv;
    long long rows;    // B * H * dv
    int vstar;         // 1: v holds beta . v
    int ipe;           // 1: I_prior is [H, dv, dk]
};

constexpr int kStepThreads = 256;

// Sum over groups of W consecutive lanes (W a power of two <= 32).
template <int W>
__device__ inline float group_sum(float x) {
    if (W >= 16) x = row16_sum(x);
    else {
#pragma unroll
        for (int o = W / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    }
    if (W == 32) x += __shfl_xor(x, 16, 64);
    return x;
}

template <int DK, typename TIn, typename TOut>
__global__ __launch_bounds__(kStepThreads) void step_kernel(StepArgs a) {
    // threads per value row (4 columns each, or for wide heads 32 threads
    // walking the row in 4-wide vectors 128 columns apart: coalesced 512-byte
    // spans per vector, few registers)
    constexpr int kTPR = DK / 4 < 32 ? DK / 4 : 32;
    constexpr int kVecs = DK / (4 * kTPR);
    constexpr int kRowsPerBlock = kStepThreads / kTPR;
    const int tid = threadIdx.x;
    const long long row = (long long)blockIdx.x * kRowsPerBlock + tid / kTPR;
    const int j0 = (tid % kTPR) * 4;
    // every lane of a row group takes part in the reduction, so rows past the
    // end are clamped (and not stored) instead of returning early
    const bool valid = row < a.rows;
    const long long r = valid ? row : a.rows - 1;
    const long long bh = r / a.dv;
    const int i = (int)(r % a.dv);
    const int h = (int)(bh % a.H);

    const TIn *qp = (const TIn *)a.q + bh * DK + j0;
    const TIn *kp = (const TIn *)a.k + bh * DK + j0;
    const float bt = io<TIn>::to_f32(((const TIn *)a.beta)[bh * a.dv + i]);
    const float vv = io<TIn>::to_f32(((const TIn *)a.v)[bh * a.dv + i]);
    const float bv = a.vstar ? vv : bt * vv;
    const float2 gc = gate(a.A[h], io<TIn>::to_f32(((const TIn *)a.dt)[bh]), a.ipe ? 1.f : a.Ip[h]);
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < kVecs; ++m) {
        const int jm = 4 * kTPR * m;                       // column offset of this vector
        float qq[4], kk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) { qq[e] = io<TIn>::to_f32(qp[jm + e]); kk[e] = io<TIn>::to_f32(kp[jm + e]); }
        // c per entry: (1 - alpha) I_prior[h] or (1 - alpha) I_prior[h, i, j]
        float cc[4] = {gc.y, gc.y, gc.y, gc.y};
        if (a.ipe) {
            const f32x4 ip4 = *(const f32x4 *)(a.Ip + ((size_t)h * a.dv + i) * DK + j0 + jm);
#pragma unroll
            for (int e = 0; e < 4; ++e) cc[e] = gc.y * ip4[e];
        }
        f32x4 *mup = (f32x4 *)(a.mu + r * DK + j0 + jm);
        f32x4 *Ipp = (f32x4 *)(a.I + r * DK + j0 + jm);
        const f32x4 mu4 = __builtin_nontemporal_load(mup);
        const f32x4 I4 = __builtin_nontemporal_load(Ipp);
        float mun[4], In[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            In[e] = fmaf(gc.x, I4[e], fmaf(bt, kk[e] * kk[e], cc[e]));
            const float num = fmaf(gc.x * I4[e], mu4[e], bv * kk[e]);   // alpha I mu + beta v k
            mun[e] = num / In[e];
            acc = fmaf(mun[e], qq[e], acc);
        }
        if (valid) {
            __builtin_nontemporal_store(f32x4{mun[0], mun[1], mun[2], mun[3]}, mup);
            __builtin_nontemporal_store(f32x4{In[0], In[1], In[2], In[3]}, Ipp);
        }
    }
    const float yv = group_sum<kTPR>(acc);
    if (valid && tid % kTPR == 0)
        ((TOut *)a.y)[r] = io<TOut>::from_f32(yv);
}

// ---------------------------------------------------------------------------
// backward of the frozen-importance recurrence on the matrix cores
// ---------------------------------------------------------------------------
//
// Reverse mode of S_t = a_t S_{t-1} + w_t (x) k_t, y_t = S_t q_t (w_t = beta_t .
// v_t / I_prior, a_t = e^{l_t}, l_t = -A dt_t), chunked over 64 tokens.  Inside
// a chunk, with L_t the inclusive prefix sum of l and Lam = L_63, the state and
// its adjoint G_t = dLoss/dS_t are
//     S_t = e^{L_t} S_0 + sum_{s<=t} e^{L_t - L_s} w_s k_s^T
//     G_t = e^{Lam - L_t} G_E + sum_{u>=t} e^{L_u - L_t} gy_u q_u^T
// where S_0 is the state before the chunk and G_E the adjoint of the state
// after it.  Each gradient is then one product with a boundary matrix plus one
// causal, decay-weighted product inside the chunk:
//     gq_t = e^{L_t} S_0^T gy_t + sum_{s<=t} e^{L_t - L_s} (gy_t . w_s) k_s
//     gk_s = e^{Lam - L_s} G_E^T w_s + sum_{t>=s} e^{L_t - L_s} (gy_t . w_s) q_t
//     gw_s = e^{Lam - L_s} G_E k_s + sum_{t>=s} e^{L_t - L_s} (q_t . k_s) gy_t
// and, since every term's decay exponent is a difference of prefix sums,
//     dLoss/dl_s = sum_{t>=s in the chunk} (q_t . gq_t - k_t . gk_t) + <G_E, S_end>,
// which is taken in the equal form without the large cancelling pair
// <G_E, S_end> - sum k . (G_E part of gk):
//     dLoss/dl_s = e^{Lam} <G_E, S_0> + sum_{r<s} k_r . gkE_r
//                  + sum_{t>=s} (q_t . gq_t - k_t . gkI_t)
// (gkE, gkI: the G_E and the in-chunk parts of gk).
// The chunk boundaries follow from the chunks' own contributions
//     dS_c = sum_s e^{Lam - L_s} w_s k_s^T,   dG_c = sum_t e^{L_t} gy_t q_t^T
// as S_0(c+1) = e^{Lam_c} S_0(c) + dS_c and G_E(c-1) = e^{Lam_c} G_E(c) + dG_c.
// fzb_state_kernel walks the chunks in order for both (the state forward, the
// adjoint backward, side by side), fzb_grad_kernel forms the gradients of
// every chunk at once, fzb_head_kernel sums gA and gI_prior over the batch.
//
// Products take bf16 operands with fp32 accumulation (as the frozen forward);
// the boundary matrices are handed from the state walk to the gradient kernel
// in bf16.


constexpr int kFbC = 64;                  // tokens per chunk

struct FzbArgs {
    const bf16_t *q, *k, *v, *beta, *dt;  // beta NULL: v holds the write beta . v
    const void *gy;
    const float *A, *Ip, *mu0, *gmuT;
    float *gq, *gk, *gv, *gbeta, *gdt, *gA, *gIp, *gmu0;
    // workspace, per (b, h, chunk): S0T [DK][DV], GE [DV][DK], GT [DK][DV] (bf16),
    // pA, pI (float)
    bf16_t *sT, *ge, *gT;
    float *pA, *pI;
    int B, T, H, nc;
    int vec_g;                            // gv and gbeta 16-byte aligned: vector stores
};

// Fragment of a 16x16x32 MFMA operand whose k index runs along the rows of a
// row-major LDS array X (row stride rs): lane l gets X[k0 + 8 (l/16) + e][c0 + l%16],
// e = 0..7, through two LDS transpose loads (within a 16-lane group, lane m
// receives element m%4 of the 8-byte loads of lanes 4e + m/4).
__device__ inline bf16x8_t lds_trfrag(const bf16_t *X, int rs, int k0, int c0, int lane) {
    const int g = lane >> 4, m = lane & 15;
    const bf16_t *p = X + (k0 + 8 * g + (m >> 2)) * rs + c0 + 4 * (m & 3);
    typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 4 * rs));
    return cat8(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi));
}
// Fragment whose k index runs along a row: lane l gets X[r0 + l%16][k0 + 8 (l/16) + e].
__device__ inline bf16x8_t rowfrag(const bf16_t *X, int rs, int r0, int k0, int lane) {
    return *(const bf16x8_t *)(X + (r0 + (lane & 15)) * rs + k0 + 8 * (lane >> 4));
}
__device__ inline f32x4 mfma16(bf16x8_t a, bf16x8_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline uint2 pack4_bf16(f32x4 x) { return make_uint2(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])); }
// Fragment-major layout of a [DK][DV] boundary matrix (S_0^T, G_E^T): the A
// operand of rows 16 jb and columns 32 f (lane l: row 16 jb + l % 16, columns
// 32 f + 8 (l / 16) .. + 7) is 64 lanes x 16 bytes, contiguous, so that the
// state walk's stores and the gradient kernel's loads are whole 512-byte runs.
__device__ inline size_t fragidx(int dv, int jb, int f, int lane) {
    return ((size_t)(jb * (dv / 32) + f) * 64 + lane) * 8;
}

__device__ inline u32x4 pack8_bf16(const float *x) {
    return u32x4{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
}

// Inclusive prefix sum L of l_t = -A dt_t over the chunk, lane = token (l = 0
// past the end of the sequence; every wave forms it), in two steps so that the
// load can be issued early: the raw bits of dt for token t0 + lane (clamped to
// the last token), then the scan.
__device__ inline uint32_t fzb_dt_bits(const FzbArgs &a, size_t seq, int t0, int lane) {
    return __builtin_bit_cast(uint16_t, a.dt[seq + (size_t)min(t0 + lane, a.T - 1) * a.H]);
}
__device__ inline float fzb_lam_bits(const FzbArgs &a, uint32_t bits, int t0, int lane, float Ah) {
    const float l = t0 + lane < a.T ? -Ah * __uint_as_float(bits << 16) : 0.f;
    return wave_incl_scan(l, lane);
}

template <int DK, int DV>
struct FzbLds {
    // rows padded by 8 elements (16 bytes), so that the 16 rows a fragment read
    // touches start in different banks
    static constexpr int kRK = DK + 8, kRV = DV + 8, kRP = kFbC + 8;   // row strides (bf16)
    static constexpr int kQ = 0, kK = kQ + kFbC * kRK, kG = kK + kFbC * kRK, kW = kG + kFbC * kRV;
    static constexpr int kP = kW + kFbC * kRV;            // one score matrix [64][kRP]
    static constexpr int kGradHalves = kP + kFbC * kRP;
    static constexpr int kL = kGradHalves * 2;            // L of the chunk's tokens [64] (float)
    static constexpr int kGradBytes = kL + kFbC * 4;
    // fzb_grad's closing sums (per-wave token sums of q.gq, k.gkI, k.gkE, and
    // of gw.w and <G_E, S_0>) reuse the score matrix's space
    static_assert((3 * 4 * kFbC + 8) * 4 <= kFbC * kRP * 2, "closing sums exceed the score buffer");
};

// Stage the chunk's Q, K, gy and w = beta v / I_prior (bf16, rows = tokens);
// zeros past the end of the sequence.
template <int DK, int DV, typename TG>
__device__ inline void fzb_stage(const FzbArgs &a, bf16_t *hb, size_t seq, int t0, float inv_ip, int tid) {
    using L = FzbLds<DK, DV>;
    constexpr int kPk = DK / 8, kPv = DV / 8;
    constexpr int NQ = kFbC * kPk / 256, NV = kFbC * kPv / 256;   // packets per thread
    constexpr int kGP = sizeof(TG) / 2;                             // 16-byte packets per 8 values of gy
    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
    // the loads of each half (q, k; then v, beta, gy) first, so that they are
    // in flight together (rows past the end clamped to the last token, zeroed
    // at the commit)
    const int tl = a.T - 1;
    {
        u32x4 qv[NQ], kv[NQ];
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            const int p = tid + 256 * n, t = p / kPk, col = 8 * (p % kPk);
            const size_t o = (seq + (size_t)min(t0 + t, tl) * a.H) * DK + col;
            qv[n] = *(const u32x4 *)(a.q + o);
            kv[n] = *(const u32x4 *)(a.k + o);
        }
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            const int p = tid + 256 * n, t = p / kPk, col = 8 * (p % kPk);
            const bool ok = t0 + t < a.T;
            *(u32x4 *)(hb + L::kQ + t * L::kRK + col) = ok ? qv[n] : z;
            *(u32x4 *)(hb + L::kK + t * L::kRK + col) = ok ? kv[n] : z;
        }
    }
    u32x4 vv[NV], bv[NV], gv[NV][kGP];
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        const int p = tid + 256 * n, t = p / kPv, col = 8 * (p % kPv);
        const size_t o = (seq + (size_t)min(t0 + t, tl) * a.H) * DV + col;
        vv[n] = *(const u32x4 *)(a.v + o);
        bv[n] = a.beta ? *(const u32x4 *)(a.beta + o) : z;
#pragma unroll
        for (int x = 0; x < kGP; ++x) gv[n][x] = *(const u32x4 *)((const TG *)a.gy + o + 4 * x);
    }
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        const int p = tid + 256 * n, t = p / kPv, col = 8 * (p % kPv);
        const bool ok = t0 + t < a.T;
        float g[8], w[8];
        if (kGP == 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) { g[2 * i] = bf_lo(gv[n][0][i]); g[2 * i + 1] = bf_hi(gv[n][0][i]); }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) g[i] = __uint_as_float(gv[n][i / 4 % kGP][i % 4]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[2 * i] = bf_lo(vv[n][i]);
            w[2 * i + 1] = bf_hi(vv[n][i]);
            if (a.beta) {
                w[2 * i] *= bf_lo(bv[n][i]);
                w[2 * i + 1] *= bf_hi(bv[n][i]);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            g[i] = ok ? g[i] : 0.f;
            w[i] = ok ? w[i] * inv_ip : 0.f;
        }
        *(u32x4 *)(hb + L::kG + t * L::kRV + col) = pack8_bf16(g);
        *(u32x4 *)(hb + L::kW + t * L::kRV + col) = pack8_bf16(w);
    }
}

// The chunk-boundary states and adjoints, one workgroup per (b, h, 64 value
// rows, half of the key channels) and direction, walking the chunks in order
// (the chain of a chunk step is short, so more and smaller walks overlap
// better on a CU; the key halves of a row block read the same w or gy, from
// L2): the first half of the grid
// runs the state forward, S_0(c+1) = e^{Lam_c} S_0(c) + sum_s e^{Lam_c - L_s} w_s k_s^T
// from mu0, writing S_0(c)^T; the second half runs the adjoint backward,
// G_E(c-1) = e^{Lam_c} G_E(c) + sum_t e^{L_t} gy_t q_t^T from gmuT, writing G_E(c)^T
// and (through LDS) G_E(c), and finally gmu0 = G_E(-1).  The running matrix stays
// in fp32 MFMA accumulators: wave w owns rows 16 w.. of the workgroup's 64 and
// its KJ key channels.  Each chunk's inputs are loaded into registers while the
// chunk before it computes.
constexpr int kFzsKS = 2;                                 // key-channel splits of the state walk
template <int DK, int DV>
struct FzsLds {
    static constexpr int KJ = DK / kFzsKS;                // key channels per workgroup
    static constexpr int kRK = KJ + 8, kRW = 64 + 8;     // row strides (bf16)
    static constexpr int kK = 0;                          // K or Q, the workgroup's channels [64 tokens][KJ]
    static constexpr int kW = kK + kFbC * kRK;            // w or gy, the workgroup's rows [64 tokens][64]
    static constexpr int kT = kW + kFbC * kRW;            // G_E transpose tile [64 rows][KJ]
    static constexpr int kBytes = (kT + 64 * kRK) * 2;
};

template <int DK, int DV, typename TG>
__global__ __launch_bounds__(256) void fzb_state_kernel(FzbArgs a) {
    using L = FzsLds<DK, DV>;
    constexpr int KJ = L::KJ;
    static_assert(KJ % 32 == 0 && kFbC * KJ / 8 % 256 == 0, "key channels per state walk");
    constexpr int RBH = DV / 64;                          // row blocks per head
    constexpr int NQ = kFbC * KJ / 8 / 256;               // 16-byte packets of K or Q per thread
    constexpr int kGP = sizeof(TG) / 2;                   // 16-byte packets per 8 values of gy
    extern __shared__ float lds_f[];
    bf16_t *hb = (bf16_t *)lds_f;
    const int n_half = a.B * a.H * RBH * kFzsKS;
    int wg = blockIdx.x;
    const bool adj = wg >= n_half;                        // second half of the grid: the adjoint
    if (adj) wg -= n_half;
    // the blocks of a head read the same keys or queries and rows: keep them on one XCD
    if (n_half % 8 == 0) wg = (wg % 8) * (n_half / 8) + wg / 8;
    const int bh = wg / (RBH * kFzsKS), i0 = 64 * (wg / kFzsKS % RBH), j0 = KJ * (wg % kFzsKS);
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    const size_t seq = (size_t)b * a.T * a.H + h;
    const float Ah = a.A[h], inv_ip = 1.f / a.Ip[h];
    const int nc = a.nc, tl = a.T - 1;
    const size_t st = (size_t)bh * DV * DK;
    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
    // the running matrix, D layout: lane holds rows i0 + 16 w + 4 g + r of key channel j0 + 16 jb + m
    f32x4 S[KJ / 16];
    {
        const float *init = adj ? a.gmuT : a.mu0;
#pragma unroll
        for (int jb = 0; jb < KJ / 16; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[jb][r] = init ? init[st + (size_t)(i0 + 16 * w + 4 * g + r) * DK + j0 + 16 * jb + m] : 0.f;
    }
    // prefetch registers, two chunks' worth: K or Q packets, and per row packet
    // two 16-byte words, (v, beta) for the state or gy (bf16: one word, fp32: two)
    u32x4 pk0[NQ], px0[2][2], pk1[NQ], px1[2][2];
    uint32_t pd0 = 0, pd1 = 0;                            // dt bits of the lane's token
    // Every prefetch is one unconditional load from an address chosen by
    // pointer selects: a load under a branch, or a select between a loaded
    // value and a constant, makes the compiler wait for it at once (to copy
    // it into the merged register), which would undo the two-chunk lead.
    // Packets that the commit does not use (beta absent, bf16 gy) repeat the
    // first one.
    const char *kq_base = adj ? (const char *)a.q : (const char *)a.k;
    const char *x0_base = adj ? (const char *)a.gy : (const char *)a.v;
    const size_t x0_esz = adj ? sizeof(TG) : sizeof(bf16_t);
    const char *x1_base = adj ? (kGP == 2 ? x0_base + 4 * sizeof(TG) : x0_base)
                              : (a.beta ? (const char *)a.beta : x0_base);
    auto load = [&](int c, u32x4 (&pk)[NQ], u32x4 (&px)[2][2], uint32_t &pd) __attribute__((always_inline)) {
        const int t0 = c * kFbC;
        pd = fzb_dt_bits(a, seq, t0, lane);
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            const int p = tid + 256 * n, t = p / (KJ / 8), col = 8 * (p % (KJ / 8));
            const size_t o = (seq + (size_t)min(t0 + t, tl) * a.H) * DK + j0 + col;
            pk[n] = *(const u32x4 *)(kq_base + o * sizeof(bf16_t));
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int p = tid + 256 * n, t = p / 8, col = 8 * (p % 8);
            const size_t o = (seq + (size_t)min(t0 + t, tl) * a.H) * DV + i0 + col;
            px[n][0] = *(const u32x4 *)(x0_base + o * x0_esz);
            px[n][1] = *(const u32x4 *)(x1_base + o * x0_esz);
        }
    };
    auto commit = [&](int c, float Lt, float Lam, const u32x4 (&pk)[NQ], const u32x4 (&px)[2][2])
                      __attribute__((always_inline)) {
        const int t0 = c * kFbC;
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            const int p = tid + 256 * n, t = p / (KJ / 8), col = 8 * (p % (KJ / 8));
            *(u32x4 *)(hb + L::kK + t * L::kRK + col) = (t0 + t < a.T) ? pk[n] : z;
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int p = tid + 256 * n, t = p / 8, col = 8 * (p % 8);
            const bool ok = t0 + t < a.T;
            const float lt = __shfl(Lt, t, 64);
            float x[8];
            if (adj) {
                const float f = __expf(lt);                       // gy scaled by e^{L_t}
                if (kGP == 1) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) { x[2 * i] = bf_lo(px[n][0][i]); x[2 * i + 1] = bf_hi(px[n][0][i]); }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        x[i] = __uint_as_float(px[n][0][i]);
                        x[4 + i] = __uint_as_float(px[n][1][i]);
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] = ok ? x[i] * f : 0.f;
            } else {
                const float f = __expf(Lam - lt) * inv_ip;        // w = beta v / I_prior scaled by e^{Lam - L_t}
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v0 = bf_lo(px[n][0][i]), v1 = bf_hi(px[n][0][i]);
                    if (a.beta) { v0 *= bf_lo(px[n][1][i]); v1 *= bf_hi(px[n][1][i]); }
                    x[2 * i] = ok ? v0 * f : 0.f;
                    x[2 * i + 1] = ok ? v1 * f : 0.f;
                }
            }
            *(u32x4 *)(hb + L::kW + t * L::kRW + col) = pack8_bf16(x);
        }
    };
    auto step = [&](int n, u32x4 (&pk)[NQ], u32x4 (&px)[2][2], uint32_t &pd) __attribute__((always_inline)) {
        const int c = adj ? nc - 1 - n : n;
        const size_t cb = (size_t)bh * nc + c;
        const float Lt = fzb_lam_bits(a, pd, c * kFbC, lane, Ah);
        const float Lam = wave_read(Lt, 63);
        __syncthreads();                                  // the previous chunk's reads of LDS are done
        commit(c, Lt, Lam, pk, px);
        __syncthreads();
        // the boundary matrix of chunk c, before this chunk's update: S_0(c)^T or
        // G_E(c)^T, fragment-major.  Lane (g, m) holds rows 4 g .. 4 g + 3 (of the
        // wave's 16) of key columns 16 jb + m; a swap with lane (g ^ 1, m) over
        // two key blocks leaves 8 consecutive rows of one key column in each
        // lane: block jb in the even-g lane, jb + 1 in the odd one.
        {
            bf16_t *dst = (adj ? a.gT : a.sT) + cb * DK * DV;
            const int f = i0 / 32 + (w >> 1), fl = 16 * (2 * (w & 1) + (g >> 1)) + m;
#pragma unroll
            for (int jb = 0; jb < KJ / 16; jb += 2) {
                const uint2 p0 = pack4_bf16(S[jb]), p1 = pack4_bf16(S[jb + 1]);
                const auto x = __builtin_amdgcn_permlane16_swap(p0.x, p1.x, false, false);
                const auto y = __builtin_amdgcn_permlane16_swap(p0.y, p1.y, false, false);
                *(uint4 *)(dst + fragidx(DV, j0 / 16 + jb + (g & 1), f, fl)) = make_uint4(x[0], y[0], x[1], y[1]);
            }
            if (adj) {
                // G_E(c) row-major: through LDS, rows of the workgroup's 64
#pragma unroll
                for (int jb = 0; jb < KJ / 16; ++jb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        hb[L::kT + (16 * w + 4 * g + r) * L::kRK + 16 * jb + m] = (bf16_t)S[jb][r];
            }
        }
        // update: S = e^{Lam} S + (rows of W or G)^T (K or Q), k = tokens
        const float e = __expf(Lam);
        const bf16x8_t a0 = lds_trfrag(hb + L::kW, L::kRW, 0, 16 * w, lane);
        const bf16x8_t a1 = lds_trfrag(hb + L::kW, L::kRW, 32, 16 * w, lane);
#pragma unroll
        for (int jb = 0; jb < KJ / 16; ++jb) {
            f32x4 x = S[jb] * e;
            x = mfma16(a0, lds_trfrag(hb + L::kK, L::kRK, 0, 16 * jb, lane), x);
            S[jb] = mfma16(a1, lds_trfrag(hb + L::kK, L::kRK, 32, 16 * jb, lane), x);
        }
        // the loads two chunks ahead, issued after the boundary stores and the
        // products: right after the barrier every wave of the CU would queue
        // its loads and stores at once and wait for the address units
        if (n + 2 < nc) load(adj ? c - 2 : c + 2, pk, px, pd);
        if (adj) {
            __syncthreads();
            bf16_t *gep = a.ge + cb * DV * DK;
            for (int p = tid; p < 64 * KJ / 8; p += 256) {
                const int r = p / (KJ / 8), col = 8 * (p % (KJ / 8));
                *(u32x4 *)(gep + (size_t)(i0 + r) * DK + j0 + col) = *(const u32x4 *)(hb + L::kT + r * L::kRK + col);
            }
        }
    };
    if (nc > 0) load(adj ? nc - 1 : 0, pk0, px0, pd0);
    if (nc > 1) load(adj ? nc - 2 : 1, pk1, px1, pd1);
    for (int n = 0; n < nc; n += 2) {
        step(n, pk0, px0, pd0);
        if (n + 1 < nc) step(n + 1, pk1, px1, pd1);
    }
    if (adj && a.gmu0) {
#pragma unroll
        for (int jb = 0; jb < KJ / 16; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r) a.gmu0[st + (size_t)(i0 + 16 * w + 4 * g + r) * DK + j0 + 16 * jb + m] = S[jb][r];
    }
}

// One workgroup per (b, h, chunk): the gradients of the chunk's tokens, and
// the chunk's shares of gA and of sum gw . w (for gI_prior).  Two workgroups
// share a CU (LDS under half of it), so that one's loads overlap the other's
// products.  Order: stage; scores q.k into P; the gw blocks; scores gy.w into
// P; the gq and gk blocks; the closing sums.
template <int DK, int DV, typename TG>
__global__ __launch_bounds__(256, 2) void fzb_grad_kernel(FzbArgs a) {
    using L = FzbLds<DK, DV>;
    extern __shared__ float lds_f[];
    bf16_t *hb = (bf16_t *)lds_f;
    bf16_t *P = hb + L::kP;
    const int bh = blockIdx.x / a.nc, c = blockIdx.x % a.nc;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    const size_t seq = (size_t)b * a.T * a.H + h;
    const int t0 = c * kFbC;
    const float Ah = a.A[h], inv_ip = 1.f / a.Ip[h];
    const uint32_t dtb = fzb_dt_bits(a, seq, t0, lane);   // issued before the staging loads
    // v and beta as the gw blocks use them (block x: rows 16 (w + 4 x) + 4 g..,
    // the lane's token 16 sb + m), loaded with the staging loads and kept in
    // registers where that leaves room, so that the gw blocks wait for no load
    // (loaded there, each 16-token block waited for its own)
    constexpr bool kPre = DV <= 128;
    constexpr int NIP = kPre ? DV / 64 : 1;
    uint2 vq[NIP][4], bq[NIP][4];
    if constexpr (kPre) {
        const bf16_t *bsrc = a.beta ? a.beta : a.v;           // no beta: not read
#pragma unroll
        for (int x = 0; x < NIP; ++x)
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                const size_t o = (seq + (size_t)min(t0 + 16 * sb + m, a.T - 1) * a.H) * DV + 16 * (w + 4 * x) + 4 * g;
                vq[x][sb] = *(const uint2 *)(a.v + o);
                bq[x][sb] = *(const uint2 *)(bsrc + o);
            }
    }
    fzb_stage<DK, DV, TG>(a, hb, seq, t0, inv_ip, tid);
    const float Lt = fzb_lam_bits(a, dtb, t0, lane, Ah);  // L of token `lane`
    const float Lam = wave_read(Lt, 63);
    // L in LDS as well (read after the first barrier): a token's L is then one
    // read, four consecutive tokens' one 16-byte read, not lane shuffles
    const float *Ls = (const float *)((const char *)hb + L::kL);
    if (w == 0) ((float *)Ls)[lane] = Lt;

    // The output blocks of wave w: first its NI value blocks ib = w + 4 x (gw;
    // A operand G_E rows 16 ib), then for each of its NJ key blocks jb = w + 4 x
    // a gq and a gk block (A operands S_0^T and G_E^T rows 16 jb).  The A
    // fragments come from HBM; each block's are loaded while the block before
    // it computes (the first ones during the scores).
    constexpr int NJ = DK / 64, NI = DV / 64, NB = NI + 2 * NJ, NF = (DK > DV ? DK : DV) / 32;
    const size_t cb = (size_t)blockIdx.x;
    const bf16_t *s0t = a.sT + cb * DK * DV, *gtp = a.gT + cb * DK * DV, *gep = a.ge + cb * DV * DK;
    auto load_block = [&](int n, bf16x8_t *dst) __attribute__((always_inline)) {
        if (n < NI) {
#pragma unroll
            for (int f = 0; f < DK / 32; ++f) dst[f] = rowfrag(gep, DK, 16 * (w + 4 * n), 32 * f, lane);
        } else {
            const int x = n - NI;
            const bf16_t *base = (x & 1) ? gtp : s0t;
#pragma unroll
            for (int f = 0; f < DV / 32; ++f)
                dst[f] = *(const bf16x8_t *)(base + fragidx(DV, w + 4 * (x >> 1), f, lane));
        }
    };
    bf16x8_t fr[2][NF];
    load_block(0, fr[0]);
    __syncthreads();

    // decay-masked scores into P, bf16 as [t][s]: e^{L_t - L_s} (rows(t) . cols(s))
    // for s <= t, 0 above
    auto scores = [&](int oa, int ob, int rs, int nk) __attribute__((always_inline)) {
        for (int n = w; n < 16; n += 4) {
            const int tb = n >> 2, sb = n & 3;
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
            if (sb <= tb) {
                for (int kk = 0; kk < nk; ++kk)
                    acc = mfma16(rowfrag(hb + oa, rs, 16 * tb, 32 * kk, lane), rowfrag(hb + ob, rs, 16 * sb, 32 * kk, lane),
                                 acc);
                const int s = 16 * sb + m;
                const float ls = Ls[s];
                const f32x4 lt4 = *(const f32x4 *)(Ls + 16 * tb + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * tb + 4 * g + r;
                    acc[r] = s <= t ? acc[r] * __expf(lt4[r] - ls) : 0.f;
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) P[(16 * tb + 4 * g + r) * L::kRP + 16 * sb + m] = (bf16_t)acc[r];
        }
    };
    scores(L::kQ, L::kK, L::kRK, DK / 32);
    __syncthreads();

    // The lane's token in column block xb is 16 xb + m.
    float eL[4], eR[4], pq[4], pk[4], pe[4];
#pragma unroll
    for (int xb = 0; xb < 4; ++xb) {
        const float lx = Ls[16 * xb + m];
        eL[xb] = __expf(lx);
        eR[xb] = __expf(Lam - lx);
        pq[xb] = 0.f;
        pk[xb] = 0.f;
        pe[xb] = 0.f;
    }
    float pw = 0.f, pb = 0.f;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        if (n == NI) {
            // the gw blocks are done with q.k: replace it by gy.w
            __syncthreads();
            scores(L::kG, L::kW, L::kRV, DV / 32);
            __syncthreads();
        }
        const bf16x8_t *af = fr[n & 1];
        const int x = n - NI;
        if (n >= NI && (x & 1)) {
            // <G_E, S_0> over the entries of this key block (the S_0^T fragments
            // of block n-1 and the G_E^T ones line up)
#pragma unroll
            for (int f = 0; f < DV / 32; ++f)
#pragma unroll
                for (int e = 0; e < 8; ++e) pb = fmaf((float)af[f][e], (float)fr[(n + 1) & 1][f][e], pb);
        }
        if (n + 1 < NB) load_block(n + 1, fr[(n + 1) & 1]);
        if (n < NI) {
            // gw^T[i][s] = e^{Lam - L_s} sum_j G_E[i][j] k[s][j] + sum_t gy[t][i] P[t][s];
            // gv = gw beta / I_prior (v* input: gw / I_prior), gbeta = gw v / I_prior
            const int ib = w + 4 * n, i = 16 * ib + 4 * g;
            const bf16x8_t g0 = lds_trfrag(hb + L::kG, L::kRV, 0, 16 * ib, lane);
            const bf16x8_t g1 = lds_trfrag(hb + L::kG, L::kRV, 32, 16 * ib, lane);
            constexpr int kSbU = kPre ? 4 : 1;             // rolled where the registers are short
#pragma unroll kSbU
            for (int sb = 0; sb < 4; ++sb) {
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kj = 0; kj < DK / 32; ++kj)
                    acc = mfma16(af[kj], rowfrag(hb + L::kK, L::kRK, 16 * sb, 32 * kj, lane), acc);
                acc *= eR[sb];
                if (sb < 2) acc = mfma16(g0, lds_trfrag(P, L::kRP, 0, 16 * sb, lane), acc);
                acc = mfma16(g1, lds_trfrag(P, L::kRP, 32, 16 * sb, lane), acc);
                const int s = 16 * sb + m;
                const uint2 ww = *(const uint2 *)(hb + L::kW + s * L::kRV + i);
                pw += (acc[0] * bf_lo(ww.x) + acc[1] * bf_hi(ww.x)) + (acc[2] * bf_lo(ww.y) + acc[3] * bf_hi(ww.y));
                if (t0 + s < a.T) {
                    const size_t o = (seq + (size_t)(t0 + s) * a.H) * DV + i;
                    const uint2 vv = kPre ? vq[n < NIP ? n : 0][sb] : *(const uint2 *)(a.v + o);
                    const float vf[4] = {bf_lo(vv.x), bf_hi(vv.x), bf_lo(vv.y), bf_hi(vv.y)};
                    f32x4 gvv, gbb;
                    if (a.beta) {
                        const uint2 bb = kPre ? bq[n < NIP ? n : 0][sb] : *(const uint2 *)(a.beta + o);
                        const float bf[4] = {bf_lo(bb.x), bf_hi(bb.x), bf_lo(bb.y), bf_hi(bb.y)};
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float gwi = acc[r] * inv_ip;
                            gvv[r] = gwi * bf[r];
                            gbb[r] = gwi * vf[r];
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) gvv[r] = acc[r] * inv_ip;
                    }
                    if (a.vec_g) {
                        *(f32x4 *)(a.gv + o) = gvv;
                        if (a.beta) *(f32x4 *)(a.gbeta + o) = gbb;
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            a.gv[o + r] = gvv[r];
                            if (a.beta) a.gbeta[o + r] = gbb[r];
                        }
                    }
                }
            }
        } else if (!(x & 1)) {
            // gq^T[j][t] = e^{L_t} sum_i S_0^T[j][i] gy[t][i] + sum_s k[s][j] P[t][s]
            const int jb = w + 4 * (x >> 1), j = 16 * jb + 4 * g;
            const bf16x8_t k0 = lds_trfrag(hb + L::kK, L::kRK, 0, 16 * jb, lane);
            const bf16x8_t k1 = lds_trfrag(hb + L::kK, L::kRK, 32, 16 * jb, lane);
#pragma unroll 1
            for (int tb = 0; tb < 4; ++tb) {
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ki = 0; ki < DV / 32; ++ki)
                    acc = mfma16(af[ki], rowfrag(hb + L::kG, L::kRV, 16 * tb, 32 * ki, lane), acc);
                acc *= eL[tb];
                acc = mfma16(k0, rowfrag(P, L::kRP, 16 * tb, 0, lane), acc);
                if (tb >= 2) acc = mfma16(k1, rowfrag(P, L::kRP, 16 * tb, 32, lane), acc);
                const int t = 16 * tb + m;
                const uint2 qq = *(const uint2 *)(hb + L::kQ + t * L::kRK + j);
                pq[tb] += (acc[0] * bf_lo(qq.x) + acc[1] * bf_hi(qq.x)) + (acc[2] * bf_lo(qq.y) + acc[3] * bf_hi(qq.y));
                if (t0 + t < a.T) *(f32x4 *)(a.gq + (seq + (size_t)(t0 + t) * a.H) * DK + j) = acc;
            }
        } else {
            // gk^T[j][s] = e^{Lam - L_s} sum_i G_E^T[j][i] w[s][i] + sum_t q[t][j] P[t][s]
            const int jb = w + 4 * (x >> 1), j = 16 * jb + 4 * g;
            const bf16x8_t q0 = lds_trfrag(hb + L::kQ, L::kRK, 0, 16 * jb, lane);
            const bf16x8_t q1 = lds_trfrag(hb + L::kQ, L::kRK, 32, 16 * jb, lane);
#pragma unroll 1
            for (int sb = 0; sb < 4; ++sb) {
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f}, aci = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ki = 0; ki < DV / 32; ++ki)
                    acc = mfma16(af[ki], rowfrag(hb + L::kW, L::kRV, 16 * sb, 32 * ki, lane), acc);
                acc *= eR[sb];
                if (sb < 2) aci = mfma16(q0, lds_trfrag(P, L::kRP, 0, 16 * sb, lane), aci);
                aci = mfma16(q1, lds_trfrag(P, L::kRP, 32, 16 * sb, lane), aci);
                const int s = 16 * sb + m;
                const uint2 kk = *(const uint2 *)(hb + L::kK + s * L::kRK + j);
                const float k4[4] = {bf_lo(kk.x), bf_hi(kk.x), bf_lo(kk.y), bf_hi(kk.y)};
                pe[sb] += (acc[0] * k4[0] + acc[1] * k4[1]) + (acc[2] * k4[2] + acc[3] * k4[3]);
                pk[sb] += (aci[0] * k4[0] + aci[1] * k4[1]) + (aci[2] * k4[2] + aci[3] * k4[3]);
                acc += aci;
                if (t0 + s < a.T) *(f32x4 *)(a.gk + (seq + (size_t)(t0 + s) * a.H) * DK + j) = acc;
            }
        }
    }
    // closing sums, in the score buffer's space; the 4 lane groups hold the same tokens
    __syncthreads();
    float *rq = (float *)P;                              // [wave][token] sums of q . gq
    float *rk = rq + 4 * kFbC;                           // [wave][token] sums of k . gkI
    float *re = rk + 4 * kFbC;                           // [wave][token] sums of k . gkE
    float *ri = re + 4 * kFbC;                           // [wave] sums of gw . w
    float *rb = ri + 4;                                  // [wave] partial <G_E, S_0>
#pragma unroll
    for (int xb = 0; xb < 4; ++xb) {
        pq[xb] += __shfl_xor(pq[xb], 16, 64);
        pq[xb] += __shfl_xor(pq[xb], 32, 64);
        pk[xb] += __shfl_xor(pk[xb], 16, 64);
        pk[xb] += __shfl_xor(pk[xb], 32, 64);
        pe[xb] += __shfl_xor(pe[xb], 16, 64);
        pe[xb] += __shfl_xor(pe[xb], 32, 64);
        if (g == 0) {
            rq[w * kFbC + 16 * xb + m] = pq[xb];
            rk[w * kFbC + 16 * xb + m] = pk[xb];
            re[w * kFbC + 16 * xb + m] = pe[xb];
        }
    }
    pw = row16_sum(pw);
    pw += __shfl_xor(pw, 16, 64);
    pw += __shfl_xor(pw, 32, 64);
    pb = row16_sum(pb);
    pb += __shfl_xor(pb, 16, 64);
    pb += __shfl_xor(pb, 32, 64);
    if (lane == 0) {
        ri[w] = pw;
        rb[w] = pb;
    }
    __syncthreads();
    if (w == 0) {
        // dLoss/dl_t = e^{Lam} <G_E, S_0> + sum_{r<t} k_r . gkE_r + sum_{u>=t} (q_u . gq_u - k_u . gkI_u);
        // lane = token
        const float p = ((rq[lane] + rq[kFbC + lane]) + (rq[2 * kFbC + lane] + rq[3 * kFbC + lane])) -
                        ((rk[lane] + rk[kFbC + lane]) + (rk[2 * kFbC + lane] + rk[3 * kFbC + lane]));
        const float pe0 = (re[lane] + re[kFbC + lane]) + (re[2 * kFbC + lane] + re[3 * kFbC + lane]);
        const float rev = wave_incl_scan(__shfl(p, 63 - lane, 64), lane);   // lane j: sum_{u >= 63 - j} p_u
        const float pre = wave_incl_scan(pe0, lane) - pe0;                    // sum_{r < lane} pe0_r
        const float bsum = (rb[0] + rb[1]) + (rb[2] + rb[3]);
        const float dl = __shfl(rev, 63 - lane, 64) + pre + __expf(Lam) * bsum;
        float ga = 0.f;
        if (t0 + lane < a.T) {
            const size_t o = seq + (size_t)(t0 + lane) * a.H;
            a.gdt[o] = -Ah * dl;
            ga = -(float)a.dt[o] * dl;
        }
        ga = row16_sum(ga);
        ga += __shfl_xor(ga, 16, 64);
        ga += __shfl_xor(ga, 32, 64);
        if (lane == 0) {
            a.pA[cb] = ga;
            a.pI[cb] = (ri[0] + ri[1]) + (ri[2] + ri[3]);
        }
    }
}

// gA[h] and gI_prior[h] = -(1 / I_prior) sum gw . w, summed over the batch and
// the chunks: one wave per head.
__global__ __launch_bounds__(64) void fzb_head_kernel(const float *pA, const float *pI, const float *Ip, float *gA,
                                                      float *gIp, int B, int H, int nc) {
    const int h = blockIdx.x, lane = threadIdx.x;
    float sa = 0.f, si = 0.f;
    for (int n = lane; n < B * nc; n += 64) {
        const size_t o = ((size_t)(n / nc) * H + h) * nc + n % nc;
        sa += pA[o];
        si += pI[o];
    }
    sa = row16_sum(sa);
    sa += __shfl_xor(sa, 16, 64);
    sa += __shfl_xor(sa, 32, 64);
    si = row16_sum(si);
    si += __shfl_xor(si, 16, 64);
    si += __shfl_xor(si, 32, 64);
    if (lane == 0) {
        gA[h] = sa;
        gIp[h] = -si / Ip[h];
    }
}

// One decode token of the block-diagonal-precision recurrence (2x2 blocks along
// the key axis), in place on the state (mu, P), as the block-diagonal forward
// runs it for one token: per block of key channels (2j, 2j+1) of value row i,
//     h   = P mu                               (the natural parameter before the token)
//     P'  = alpha P + (1 - alpha) I_prior Id + beta_i k k^T   (on the block)
//     h'  = alpha h + beta_i v_i k,   mu' = P'^{-1} h',   y_i = sum mu' . q
// Each thread owns 4 key channels (two blocks) of one row; a row's threads sum
// its readout.
struct Bd2StepArgs {
    const void *q, *k, *v, *beta, *dt;
    const float *A, *Ip;
    float *mu, *P;      // mu [B, H, dv, dk]; P [B, H, dv, dk/2, 2, 2]
    void *y;
    int H, dv;
    long long rows;     // B * H * dv
};

template <int DK, typename TIn, typename TOut, bool I32 = false>
__global__ __launch_bounds__(kStepThreads) void bd2_step_kernel(Bd2StepArgs a) {
    constexpr int kTPR = DK / 4;                           // threads per value row
    constexpr int kRowsPerBlock = kStepThreads / kTPR;
    const int tid = threadIdx.x;
    const long long row = (long long)blockIdx.x * kRowsPerBlock + tid / kTPR;
    const int j0 = (tid % kTPR) * 4;
    // rows past the end are clamped (and not stored): every lane of a row group
    // takes part in the reduction
    const bool valid = row < a.rows;
    const long long r = valid ? row : a.rows - 1;
    long long bh;
    int i, h;
    if (I32) {
        // rows < 2^32: 32-bit division (a 64-bit one is a long software
        // sequence; 5% of the 2x2 block-diagonal step's time at B64 H32 d128)
        const unsigned r32 = (unsigned)r, dv32 = (unsigned)a.dv;
        bh = (long long)(r32 / dv32);
        i = (int)(r32 % dv32);
        h = (int)((unsigned)bh % (unsigned)a.H);
    } else {
        bh = r / a.dv;
        i = (int)(r % a.dv);
        h = (int)(bh % a.H);
    }
    const TIn *qp = (const TIn *)a.q + bh * DK + j0;
    const TIn *kp = (const TIn *)a.k + bh * DK + j0;
    const float bt = io<TIn>::to_f32(((const TIn *)a.beta)[bh * a.dv + i]);
    const float bv = bt * io<TIn>::to_f32(((const TIn *)a.v)[bh * a.dv + i]);
    const float2 gc = gate(a.A[h], io<TIn>::to_f32(((const TIn *)a.dt)[bh]), a.Ip[h]);   // alpha, (1 - alpha) I_prior
    float qq[4], kk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) { qq[e] = io<TIn>::to_f32(qp[e]); kk[e] = io<TIn>::to_f32(kp[e]); }
    f32x4 *mup = (f32x4 *)(a.mu + r * DK + j0);
    f32x4 *Pp = (f32x4 *)(a.P + (r * DK + j0) * 2);        // two blocks of (p00, p01, p10, p11)
    const f32x4 mu4 = __builtin_nontemporal_load(mup);
    const f32x4 Pa = __builtin_nontemporal_load(Pp), Pb = __builtin_nontemporal_load(Pp + 1);
    float mun[4], Pn[8], acc = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const f32x4 Pq = blk ? Pb : Pa;
        const float p00 = Pq[0], p01 = Pq[1], p11 = Pq[3];
        const float m0 = mu4[2 * blk], m1 = mu4[2 * blk + 1], k0 = kk[2 * blk], k1 = kk[2 * blk + 1];
        const float h0 = fmaf(p00, m0, p01 * m1), h1 = fmaf(p01, m0, p11 * m1);
        const float n00 = fmaf(gc.x, p00, fmaf(bt, k0 * k0, gc.y));
        const float n11 = fmaf(gc.x, p11, fmaf(bt, k1 * k1, gc.y));
        const float n01 = fmaf(gc.x, p01, bt * (k0 * k1));
        const float g0 = fmaf(gc.x, h0, bv * k0), g1 = fmaf(gc.x, h1, bv * k1);
        const float inv = 1.f / fmaf(n00, n11, -n01 * n01);
        mun[2 * blk] = fmaf(n11, g0, -n01 * g1) * inv;
        mun[2 * blk + 1] = fmaf(n00, g1, -n01 * g0) * inv;
        acc = fmaf(mun[2 * blk], qq[2 * blk], fmaf(mun[2 * blk + 1], qq[2 * blk + 1], acc));
        Pn[4 * blk] = n00; Pn[4 * blk + 1] = n01; Pn[4 * blk + 2] = n01; Pn[4 * blk + 3] = n11;
    }
    if (valid) {
        __builtin_nontemporal_store(f32x4{mun[0], mun[1], mun[2], mun[3]}, mup);
        __builtin_nontemporal_store(f32x4{Pn[0], Pn[1], Pn[2], Pn[3]}, Pp);
        __builtin_nontemporal_store(f32x4{Pn[4], Pn[5], Pn[6], Pn[7]}, Pp + 1);
    }
    const float yv = group_sum<kTPR>(acc);
    if (valid && tid % kTPR == 0)
        ((TOut *)a.y)[r] = io<TOut>::from_f32(yv);
}

// The same decode token with 4x4 blocks: a thread's 4 key channels are one
// block (P [B, H, dv, dk/4, 4, 4], upper triangle read, written in full).
template <int DK, typename TIn, typename TOut, bool I32 = false>
__global__ __launch_bounds__(kStepThreads) void bd4_step_kernel(Bd2StepArgs a) {
    constexpr int kTPR = DK / 4;
    constexpr int kRowsPerBlock = kStepThreads / kTPR;
    const int tid = threadIdx.x;
    const long long row = (long long)blockIdx.x * kRowsPerBlock + tid / kTPR;
    const int j0 = (tid % kTPR) * 4;
    const bool valid = row < a.rows;
    const long long r = valid ? row : a.rows - 1;
    long long bh;
    int i, h;
    if (I32) {
        // rows < 2^32: 32-bit division (a 64-bit one is a long software
        // sequence; 5% of the 2x2 block-diagonal step's time at B64 H32 d128)
        const unsigned r32 = (unsigned)r, dv32 = (unsigned)a.dv;
        bh = (long long)(r32 / dv32);
        i = (int)(r32 % dv32);
        h = (int)((unsigned)bh % (unsigned)a.H);
    } else {
        bh = r / a.dv;
        i = (int)(r % a.dv);
        h = (int)(bh % a.H);
    }
    const TIn *qp = (const TIn *)a.q + bh * DK + j0;
    const TIn *kp = (const TIn *)a.k + bh * DK + j0;
    const float bt = io<TIn>::to_f32(((const TIn *)a.beta)[bh * a.dv + i]);
    const float bv = bt * io<TIn>::to_f32(((const TIn *)a.v)[bh * a.dv + i]);
    const float2 gc = gate(a.A[h], io<TIn>::to_f32(((const TIn *)a.dt)[bh]), a.Ip[h]);
    float qq[4], kk[4], k2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        qq[e] = io<TIn>::to_f32(qp[e]);
        kk[e] = io<TIn>::to_f32(kp[e]);
        k2[e] = kk[e] * kk[e];
    }
    f32x4 *mup = (f32x4 *)(a.mu + r * DK + j0);
    f32x4 *Pp = (f32x4 *)(a.P + (r * DK + j0) * 4);        // the block's 16 floats
    const f32x4 mu4 = __builtin_nontemporal_load(mup);
    const f32x4 R0 = __builtin_nontemporal_load(Pp), R1 = __builtin_nontemporal_load(Pp + 1);
    const f32x4 R2 = __builtin_nontemporal_load(Pp + 2), R3 = __builtin_nontemporal_load(Pp + 3);
    float p[10] = {R0[0], R0[1], R0[2], R0[3], R1[1], R1[2], R1[3], R2[2], R2[3], R3[3]};
    // h = P mu (P symmetric from its upper triangle)
    float hh[4];
    hh[0] = fmaf(p[0], mu4[0], fmaf(p[1], mu4[1], fmaf(p[2], mu4[2], p[3] * mu4[3])));
    hh[1] = fmaf(p[1], mu4[0], fmaf(p[4], mu4[1], fmaf(p[5], mu4[2], p[6] * mu4[3])));
    hh[2] = fmaf(p[2], mu4[0], fmaf(p[5], mu4[1], fmaf(p[7], mu4[2], p[8] * mu4[3])));
    hh[3] = fmaf(p[3], mu4[0], fmaf(p[6], mu4[1], fmaf(p[8], mu4[2], p[9] * mu4[3])));
    bd4_update(p, hh, kk, k2, gc.x, gc.y, bt, bv);
    float mun[4];
    spd4_solve(p, hh, mun);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(mun[e], qq[e], acc);
    if (valid) {
        __builtin_nontemporal_store(f32x4{mun[0], mun[1], mun[2], mun[3]}, mup);
        __builtin_nontemporal_store(f32x4{p[0], p[1], p[2], p[3]}, Pp);
        __builtin_nontemporal_store(f32x4{p[1], p[4], p[5], p[6]}, Pp + 1);
        __builtin_nontemporal_store(f32x4{p[2], p[5], p[7], p[8]}, Pp + 2);
        __builtin_nontemporal_store(f32x4{p[3], p[6], p[8], p[9]}, Pp + 3);
    }
    const float yv = group_sum<kTPR>(acc);
    if (valid && tid % kTPR == 0)
        ((TOut *)a.y)[r] = io<TOut>::from_f32(yv);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

inline bool aligned_to(const void *p, size_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

// Scratch of palimpsa_fwd_chunked_noalloc: a fixed device array that each GPU
// the library runs on holds until the process ends (callers that cannot
// allocate pass no workspace).  Host code never uses the array's name as an
// address (on the host it is only a stand-in for the symbol); it uses the
// device address that hipGetSymbolAddress returns, looked up once per device
// with that device current.
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of this device's scratch (NULL and an error on failure).
void *device_scratch(palimpsa_status *st) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *st = PALIMPSA_ERR_HIP;
        return nullptr;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void *ptr = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) {
        *st = PALIMPSA_ERR_HIP;
        return nullptr;
    }
    *st = PALIMPSA_OK;
    return g_scratch_ptr[dev];
}
inline bool head_ok(int d) { return d == 32 || d == 64 || d == 128; }
// key widths of the exact forward and the decode step: up to a head as wide as
// the model (the pages' recurrent-kernel measurement goes to 2048)
inline bool fwd_dk_ok(int d) { return head_ok(d) || d == 256 || d == 512 || d == 1024 || d == 2048; }
// value rows run in blocks of 16 (64 on the frozen path), so d_v may be any
// such multiple up to 1024 (d_v = 2 d_k, the pages' value expansion, included)
inline bool dv_ok(int d) { return d >= 16 && d <= 1024 && d % 16 == 0; }
inline bool fwd_dv_ok(int d) { return d >= 16 && d <= 4096 && d % 16 == 0; }
// option bits each entry point accepts
constexpr int kFlagsOptions = PALIMPSA_VSTAR | PALIMPSA_PRIOR_PER_ENTRY;
constexpr int kFlagsFwd = kFlagsOptions | PALIMPSA_SAVE_CHECKPOINTS;
constexpr int kFlagsBwd = kFlagsOptions | PALIMPSA_CHECKPOINTS_SAVED;
inline bool dtype_ok(int t) { return t == PALIMPSA_F32 || t == PALIMPSA_BF16; }

template <int DK, int C, typename TIn, typename TOut, int MODE, bool IPE, bool CKPT = false>
palimpsa_status launch_pass(FwdArgs a, int nseg_launched, hipStream_t s) {
    a.nwg = a.nwg_seg * nseg_launched;
    a.xcd_remap = (a.nwg % 8 == 0) ? 1 : 0;
    const size_t lds = fwd_lds_bytes<DK, C>();
    auto kern = fwd_chunked_kernel<DK, C, TIn, TOut, MODE, IPE, CKPT>;
    if (lds > 64 * 1024) {
        if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return PALIMPSA_ERR_HIP;
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3(a.nwg), dim3(kThreads), lds, s, a);
    return hipGetLastError() == hipSuccess ? PALIMPSA_OK : PALIMPSA_ERR_HIP;
}

// The time split's summary pass on the matrix cores (segments 0..nseg-2).
template <int DK, typename TIn>
palimpsa_status launch_summary(FwdArgs a, hipStream_t s) {
    constexpr int kCS = DK >= 64 ? DK / 64 : 1;   // key-column slices per (segment, head, row block)
    a.nwg = a.nwg_seg * (a.nseg - 1) * kCS;
    a.xcd_remap = (a.nwg % 8 == 0) ? 1 : 0;
    const size_t lds = 2 * SumStage<DK / kCS, TIn>::kBuf;
    auto kern = summary_mfma_kernel<DK, TIn>;
    if (lds > 64 * 1024) {
        if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return PALIMPSA_ERR_HIP;
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3(a.nwg), dim3(kThreads), lds, s, a);
    return hipGetLastError() == hipSuccess ? PALIMPSA_OK : PALIMPSA_ERR_HIP;
}

// Summary pass (segments 0..nseg-2) then the replay pass (all segments).
// (the summary pass does not read the prior, so it has no IPE variant)
template <int DK, int C, typename TIn, typename TOut, bool IPE>
palimpsa_status launch_fwd_t(const FwdArgs &a, hipStream_t s) {
    if (a.nseg > 1) {
        const palimpsa_status st = launch_summary<DK, TIn>(a, s);
        if (st != PALIMPSA_OK) return st;
    }
    return launch_pass<DK, C, TIn, TOut, kReplay, IPE>(a, a.nseg, s);
}

template <int DK, typename TIn, typename TOut, bool IPE>
palimpsa_status launch_fwd_c(const FwdArgs &a, int C, hipStream_t s) {
    switch (C) {
    case 16: return launch_fwd_t<DK, 16, TIn, TOut, IPE>(a, s);
    case 32: return launch_fwd_t<DK, 32, TIn, TOut, IPE>(a, s);
    default: return launch_fwd_t<DK, 64, TIn, TOut, IPE>(a, s);
    }
}

template <int D, typename TIn, typename TOut>
palimpsa_status launch_wide(FwdArgs a, hipStream_t s) {
    const size_t lds = (size_t)2 * WideCfg<D>::kBufFloats * sizeof(float);
    auto kern = wide_fwd_kernel<D, TIn, TOut>;
    if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return PALIMPSA_ERR_HIP;
    const long long nwg = (long long)a.B * a.H * (a.dv / WideCfg<D>::kRows);
    if (nwg > 0x7fffffffLL) return PALIMPSA_ERR_UNSUPPORTED;
    a.nwg = (int)nwg;
    a.xcd_remap = (a.nwg % 8 == 0) ? 1 : 0;
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3(a.nwg), dim3(kThreads), lds, s, a);
    return hipGetLastError() == hipSuccess ? PALIMPSA_OK : PALIMPSA_ERR_HIP;
}

// Row-parallel wide-head forward: columns per lane and column slices, the
// workspace layout [column-group records][slice readouts] (256-byte aligned;
// the records are sized for float32 inputs, 14 bytes per token and column,
// bf16 ones use 9).  Taken for d_k >= 512 when d_v is a multiple of 64,
// T >= 1 and the grid covers every CU at least once; otherwise the
// column-parallel kernel runs.
struct WideRowsPlan {
    int kcl, nq;
    long long nwg;
    size_t part_off, bytes;
};
bool plan_wide_rows(int B, int T, int H, int dk, int dv, int cus, WideRowsPlan *p) {
    if (dk < 512 || T <= 0 || dv % 64 != 0) return false;
    p->kcl = dk >= 1024 ? 32 : 16;
    p->nq = dk / (p->kcl * kWrNW);
    if (p->nq > 4) return false;   // wide_sum_kernel adds at most 4 slices
    p->nwg = (long long)B * H * (dv / 64) * p->nq;
    if (p->nwg < cus || p->nwg > 0x7fffffffLL) return false;
    const size_t ntok = (size_t)B * T * H;
    static_assert(ColGroup<float>::kWords * 4 == 14 * ColGroup<float>::kCols, "float32 records: 14 B per column");
    static_assert(ColGroup<bf16_t>::kWords * 4 <= 14 * ColGroup<bf16_t>::kCols, "bf16 records fit that size");
    p->part_off = (ntok * dk * 14 + 255) / 256 * 256;
    p->bytes = p->part_off + (size_t)p->nq * ntok * dv * sizeof(float);
    return true;
}

template <int KCL, typename TIn, typename TOut>
palimpsa_status launch_wide_rows(const FwdArgs &f, int dk, const WideRowsPlan &p, void *ws, hipStream_t s) {
    WideRowsArgs a;
    a.v = f.v; a.beta = f.beta;
    a.rec = (const uint32_t *)ws;
    a.Ip = f.Ip; a.mu0 = f.mu0; a.I0 = f.I0; a.muT = f.muT; a.IT = f.IT;
    a.part = (float *)((char *)ws + p.part_off);
    a.B = f.B; a.T = f.T; a.H = f.H; a.D = dk; a.dv = f.dv; a.nq = p.nq;
    a.nwg = (int)p.nwg;
    a.xcd_remap = (a.nwg % 8 == 0) ? 1 : 0;
    const size_t ntok = (size_t)f.B * f.T * f.H;
    const size_t prep_threads = ntok * (dk / ColGroup<TIn>::kCols);
    const size_t n = ntok * f.dv;
    const size_t lds = (size_t)2 * wr_tok<KCL>() * kWrNW * 64 * sizeof(float);
    auto kern = wide_rows_kernel<KCL, TIn>;
    if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return PALIMPSA_ERR_HIP;
    if ((prep_threads + 255) / 256 > 0x7fffffffULL || (n / 4 + 255) / 256 > 0x7fffffffULL)
        return PALIMPSA_ERR_UNSUPPORTED;
    (void)hipGetLastError();
    hipLaunchKernelGGL(wide_prep_kernel<TIn>, dim3((unsigned)((prep_threads + 255) / 256)), dim3(256), 0, s,
                       (const TIn *)f.q, (const TIn *)f.k, (const TIn *)f.dt, f.A, f.Ip, (uint32_t *)ws, ntok, f.H, dk);
    hipLaunchKernelGGL(kern, dim3(a.nwg), dim3(kWrNW * 64), lds, s, a);
    hipLaunchKernelGGL(wide_sum_kernel<TOut>, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s,
                       (const float *)a.part, (TOut *)f.y, n, p.nq);
    return hipGetLastError() == hipSuccess ? PALIMPSA_OK : PALIMPSA_ERR_HIP;
}

template <typename TIn, typename TOut>
palimpsa_status launch_wide_rows_d(const FwdArgs &f, int dk, const WideRowsPlan &p, void *ws, hipStream_t s) {
    return p.kcl == 32 ? launch_wide_rows<32, TIn, TOut>(f, dk, p, ws, s)
                       : launch_wide_rows<16, TIn, TOut>(f, dk, p, ws, s);
}

// Training forward: the forward that also stores the backward's checkpoints
// (one pass, chunk 16 as the checkpoint pass, so the states are the same bits).
template <typename TIn, typename TOut>
palimpsa_status launch_fwd_ckpt(const FwdArgs &a, int dk, bool ipe, hipStream_t s) {
    switch (dk * 2 + (ipe ? 1 : 0)) {
    case 64: return launch_pass<32, 16, TIn, TOut, kReplay, false, true>(a, 1, s);
    case 65: return launch_pass<32, 16, TIn, TOut, kReplay, true, true>(a, 1, s);
    case 128: return launch_pass<64, 16, TIn, TOut, kReplay, false, true>(a, 1, s);
    case 129: return launch_pass<64, 16, TIn, TOut, kReplay, true, true>(a, 1, s);
    case 257: return launch_pass<128, 16, TIn, TOut, kReplay, true, true>(a, 1, s);
    default: return launch_pass<128, 16, TIn, TOut, kReplay, false, true>(a, 1, s);
    }
}

template <typename TIn, typename TOut>
palimpsa_status launch_fwd_d(const FwdArgs &a, int dk, int C, bool ipe, hipStream_t s) {
    switch (dk) {
    case 256: return launch_fwd_t<256, 16, TIn, TOut, false>(a, s);   // 102.6 KB of LDS at C = 16
    case 512: return launch_wide<512, TIn, TOut>(a, s);
    case 1024: return launch_wide<1024, TIn, TOut>(a, s);
    case 2048: return launch_wide<2048, TIn, TOut>(a, s);
    default: break;
    }
    switch (dk * 2 + (ipe ? 1 : 0)) {
    case 64: return launch_fwd_c<32, TIn, TOut, false>(a, C, s);
    case 65: return launch_fwd_c<32, TIn, TOut, true>(a, C, s);
    case 128: return launch_fwd_c<64, TIn, TOut, false>(a, C, s);
    case 129: return launch_fwd_c<64, TIn, TOut, true>(a, C, s);
    case 257: return launch_fwd_c<128, TIn, TOut, true>(a, C, s);
    default: return launch_fwd_c<128, TIn, TOut, false>(a, C, s);
    }
}

size_t lds_bytes_for(int dk, int C) { return (size_t)2 * C * (3 * dk + 2 * kRowsPerWG + 2) * sizeof(float); }

// Chunk actually used: the library's choice is the largest chunk (16 to 64)
// whose double-buffered staging lets three workgroups share a CU when there
// are enough workgroups to need it, else the largest that fits the device's
// LDS.  A request caps that choice (8 is raised to 16, the reduction group):
// a larger chunk than the choice would only cost occupancy, and the results
// are the same bits for every chunk.
int pick_chunk(int requested, int dk, long long nwg, size_t lds_max) {
    const size_t budget = nwg > 256 ? 54 * 1024 : lds_max;
    int C = 64;
    while (C > 16 && lds_bytes_for(dk, C) > budget) C /= 2;
    if (requested > 0) {
        const int cap = requested < 16 ? 16 : requested;
        while (C > 16 && C > cap) C /= 2;
    }
    return C;
}

int device_cus() {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
        return 256;
    return v;
}

// Time segments of the forward.  With few (head, row block) workgroups the
// GPU is under-filled, so the sequence is cut into segments that run side by
// side (a summary pass, then a replay pass).  Auto, when fewer than two
// workgroups per CU would run: R segments fill the GPU once at three
// workgroups per CU; take the largest multiple of R up to 12 (R itself when
// R > 12), so that the replay runs as whole rounds of workgroups, and a few
// of them where R is small (several rounds even out the CUs' pace: on the
// 32-head, 32k-token layer 12 segments take 4.33 ms where 3, one round,
// take 4.60).  At most 32 segments, at least 256 tokens each, and a
// workspace that fits the no-allocation entry's scratch.  Segment lengths
// are multiples of 64 tokens, so the chunk choice never moves a segment
// boundary.
struct SegPlan {
    int nseg, seg_len;
    size_t ws_bytes;
};
SegPlan plan_segments(int B, int T, int H, int dk, int dv, int segments, int cus) {
    const long long nwg_seg = (long long)B * H * (dv / kRowsPerWG);
    long long S = 1;
    if (T > 0 && segments >= 2) {
        S = segments;
    } else if (T > 0 && segments == 0 && nwg_seg < 2LL * cus) {
        const long long R = (3LL * cus) / nwg_seg;
        S = R >= 12 ? R : R * (12 / R);
        if (S > 32) S = 32;
        if (S > T / 256) S = T / 256;
        // floats per segment, an upper bound of the workspace's share
        const long long per = 2LL * B * H * dv * dk + (long long)B * H;
        const long long cap = (long long)(kNoAllocScratchBytes / sizeof(float)) / per;
        if (S > cap) S = cap;
    }
    const long long units = (T + 63) / 64;
    if (S > units) S = units;
    if (S < 1) S = 1;
    SegPlan p;
    p.seg_len = (int)(((T + S - 1) / S + 63) / 64 * 64);
    if (p.seg_len == 0) p.seg_len = 64;
    p.nseg = (int)((T + p.seg_len - 1) / p.seg_len);
    if (p.nseg < 1) p.nseg = 1;
    // (nseg - 1) summaries (M_loc, Ibar_loc, P), the start-state copy (mu0, I0)
    p.ws_bytes = p.nseg > 1 ? (((size_t)p.nseg * 2 * B * H * dv * dk + (size_t)(p.nseg - 1) * B * H) * sizeof(float))
                            : 0;
    return p;
}

size_t device_lds_max() {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 64 * 1024;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0)
        return 64 * 1024;
    return (size_t)v;
}

template <int DK>
palimpsa_status launch_frozen(const FrozenArgs &a, hipStream_t s) {
    constexpr size_t lds = FzLds<DK>::kTotal;
    static_assert(lds <= 160 * 1024, "frozen staging exceeds the CU's LDS");
    auto kern = frozen_fwd_kernel<DK>;
    if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return PALIMPSA_ERR_HIP;
    const long long grid = (long long)a.B * a.H * (a.dv / kFzRows);
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), lds, s, a);
    return hipGetLastError() == hipSuccess ? PALIMPSA_OK : PALIMPSA_ERR_HIP;
}

// Workspace of the backward, in 256-byte aligned sections (float counts):
//   ck    [B*H][nck][dv/16][dk/32][256][4]  checkpoints, nck = ceil(T / 16)
//   pqk   [dv/16][B*T*H][2 dk]              row-block partials of gq | gk
//   ps    [dv/16][B*H][T][2]                row-block partials of (da, dc)
//   gabh, gibh [B*H]                        per-sequence gate gradient sums
//   pI0   [B*H][dv/16]                      row-block sums of gI0
//   pip   [B*H][dv][dk]                     per-entry prior only: per-sequence gI_prior
struct BwdWs {
    float *ck, *pqk, *ps, *gabh, *gibh, *pI0, *pip;
    size_t bytes;
};
BwdWs plan_bwd_ws(void *base, int B, int T, int H, int dk, int dv, bool ipe) {
    const size_t nck = (size_t)(T + kCkI - 1) / kCkI, nrb = (size_t)dv / kRowsPerWG;
    const size_t bh = (size_t)B * H, bth = bh * T;
    size_t off = 0;
    auto take = [&](size_t floats) {
        const size_t o = off;
        off = (off + floats * sizeof(float) + 255) / 256 * 256;
        return o;
    };
    const size_t o_ck = take(bh * nck * 2 * dv * dk), o_pqk = take(nrb * bth * 2 * dk), o_ps = take(nrb * bth * 2);
    const size_t o_ga = take(bh), o_gi = take(bh), o_pi = take(bh * nrb);
    const size_t o_pip = ipe ? take(bh * dv * dk) : off;
    BwdWs w;
    // section pointers only exist for a real base (a size query passes none)
    char *c = (char *)base;
    auto at = [c](size_t o) { return c ? c + o : nullptr; };
    w.ck = (float *)at(o_ck); w.pqk = (float *)at(o_pqk); w.ps = (float *)at(o_ps);
    w.gabh = (float *)at(o_ga); w.gibh = (float *)at(o_gi); w.pI0 = (float *)at(o_pi);
    w.pip = ipe ? (float *)at(o_pip) : nullptr;
    w.bytes = off;
    return w;
}

template <int DK, typename TIn, typename TG, bool IPE, bool FZ = false>
palimpsa_status launch_bwd_t(const FwdArgs &fa, const BwdArgs &ba, const BwdWs &w, float *gq, float *gk,
                             float *gdt, float *gA, float *gIp, int dt_bf16, hipStream_t s) {
    if (ba.T > 0 && fa.ck) {   // ck NULL: the training forward stored the checkpoints already
        const palimpsa_status st = launch_pass<DK, 16, TIn, float, kCheckpoint, IPE>(fa, 1, s);
        if (st != PALIMPSA_OK) return st;
    }
    const size_t lds = (size_t)BwdStage<DK>::kTotal * sizeof(float);
    auto kern = bwd_kernel<DK, TIn, TG, IPE, FZ>;
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return PALIMPSA_ERR_HIP;
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3(ba.nwg), dim3(kThreads), lds, s, ba);
    const size_t bth = (size_t)ba.B * ba.T * ba.H;
    const int nrb = ba.dv / kRowsPerWG;
    if (bth > 0) {
        const size_t n4 = bth * (2 * DK / 4);
        hipLaunchKernelGGL(bwd_qk_kernel<DK>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                           (const float *)w.pqk, gq, gk, bth, nrb);
    }
    hipLaunchKernelGGL(bwd_gate_kernel, dim3(ba.B * ba.H), dim3(256), 0, s, (const float *)w.ps, ba.dt, dt_bf16,
                       ba.A, ba.Ip, IPE ? 1 : 0, FZ ? 1 : 0, gdt, w.gabh, w.gibh, ba.B, ba.T, ba.H, nrb);
    hipLaunchKernelGGL(bwd_head_kernel, dim3((ba.H + 63) / 64), dim3(64), 0, s, (const float *)w.gabh,
                       (const float *)w.gibh, (const float *)w.pI0, ba.Ip, gA, gIp, ba.B, ba.H, nrb,
                       (ba.mu0 || FZ) ? 0 : 1, IPE ? 1 : 0, FZ ? 1 : 0);
    if (IPE) {
        const size_t per_b = (size_t)ba.H * ba.dv * DK;
        hipLaunchKernelGGL(bwd_prior_kernel, dim3((unsigned)((per_b / 4 + 255) / 256)), dim3(256), 0, s,
                           (const float *)w.pip, gIp, ba.B, per_b);
    }
    return hipGetLastError() == hipSuccess ? PALIMPSA_OK : PALIMPSA_ERR_HIP;
}

template <typename TIn, typename TG>
palimpsa_status launch_bwd_fz_d(int dk, const FwdArgs &fa, const BwdArgs &ba, const BwdWs &w, float *gq, float *gk,
                                float *gdt, float *gA, float *gIp, int dt_bf16, hipStream_t s) {
    switch (dk) {
    case 32: return launch_bwd_t<32, TIn, TG, false, true>(fa, ba, w, gq, gk, gdt, gA, gIp, dt_bf16, s);
    case 64: return launch_bwd_t<64, TIn, TG, false, true>(fa, ba, w, gq, gk, gdt, gA, gIp, dt_bf16, s);
    default: return launch_bwd_t<128, TIn, TG, false, true>(fa, ba, w, gq, gk, gdt, gA, gIp, dt_bf16, s);
    }
}

// Workspace of the matrix-core frozen backward (per (b, h, chunk), 256-byte
// aligned sections): S_0^T and G_E^T [DK][DV] and G_E [DV][DK] in bf16, and the
// chunk's gA and gw . w sums in float.  It is never larger
// than plan_bwd_ws for the same sizes (checked by the caller).
struct FzbWs {
    bf16_t *sT, *ge, *gT;
    float *pA, *pI;
    size_t bytes;
};
FzbWs plan_fzb_ws(void *base, int B, int T, int H, int dk, int dv) {
    const size_t nc = (size_t)(T + kFbC - 1) / kFbC, bhc = (size_t)B * H * nc, e = (size_t)dv * dk;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = (off + bytes + 255) / 256 * 256;
        return o;
    };
    const size_t o_s = take(bhc * e * 2), o_g = take(bhc * e * 2), o_t = take(bhc * e * 2);
    const size_t o_a = take(bhc * 4), o_i = take(bhc * 4);
    // section pointers only exist for a real base (a size query passes none)
    char *c = (char *)base;
    auto at = [c](size_t o) { return c ? c + o : nullptr; };
    FzbWs w;
    w.sT = (bf16_t *)at(o_s); w.ge = (bf16_t *)at(o_g); w.gT = (bf16_t *)at(o_t);
    w.pA = (float *)at(o_a); w.pI = (float *)at(o_i);
    w.bytes = off;
    return w;
}

template <int DK, int DV, typename TG>
palimpsa_status launch_fzb(const FzbArgs &a, hipStream_t s) {
    using L = FzbLds<DK, DV>;
    static_assert(L::kGradBytes <= 160 * 1024, "frozen backward staging exceeds the CU's LDS");
    const size_t bhc = (size_t)a.B * a.H * a.nc;
    (void)hipGetLastError();
    {
        using LS = FzsLds<DK, DV>;
        hipLaunchKernelGGL((fzb_state_kernel<DK, DV, TG>), dim3((unsigned)(2 * (size_t)a.B * a.H * (DV / 64) * kFzsKS)), dim3(256),
                           LS::kBytes, s, a);
    }
    if (bhc > 0) {
        auto k3 = fzb_grad_kernel<DK, DV, TG>;
        if (hipFuncSetAttribute((const void *)k3, hipFuncAttributeMaxDynamicSharedMemorySize, L::kGradBytes) != hipSuccess)
            return PALIMPSA_ERR_HIP;
        hipLaunchKernelGGL(k3, dim3((unsigned)bhc), dim3(256), L::kGradBytes, s, a);
    }
    hipLaunchKernelGGL(fzb_head_kernel, dim3(a.H), dim3(64), 0, s, (const float *)a.pA, (const float *)a.pI,
                       a.Ip, a.gA, a.gIp, a.B, a.H, a.nc);
    return hipGetLastError() == hipSuccess ? PALIMPSA_OK : PALIMPSA_ERR_HIP;
}

template <typename TG>
palimpsa_status launch_fzb_d(int dk, int dv, const FzbArgs &a, hipStream_t s) {
    if (dk == 64) {
        if (dv == 64) return launch_fzb<64, 64, TG>(a, s);
        return dv == 128 ? launch_fzb<64, 128, TG>(a, s) : launch_fzb<64, 256, TG>(a, s);
    }
    if (dv == 64) return launch_fzb<128, 64, TG>(a, s);
    return dv == 128 ? launch_fzb<128, 128, TG>(a, s) : launch_fzb<128, 256, TG>(a, s);
}

template <typename TIn, typename TG>
palimpsa_status launch_bwd_d(int dk, bool ipe, const FwdArgs &fa, const BwdArgs &ba, const BwdWs &w, float *gq,
                             float *gk, float *gdt, float *gA, float *gIp, int dt_bf16, hipStream_t s) {
    switch (dk * 2 + (ipe ? 1 : 0)) {
    case 64: return launch_bwd_t<32, TIn, TG, false>(fa, ba, w, gq, gk, gdt, gA, gIp, dt_bf16, s);
    case 65: return launch_bwd_t<32, TIn, TG, true>(fa, ba, w, gq, gk, gdt, gA, gIp, dt_bf16, s);
    case 128: return launch_bwd_t<64, TIn, TG, false>(fa, ba, w, gq, gk, gdt, gA, gIp, dt_bf16, s);
    case 129: return launch_bwd_t<64, TIn, TG, true>(fa, ba, w, gq, gk, gdt, gA, gIp, dt_bf16, s);
    case 257: return launch_bwd_t<128, TIn, TG, true>(fa, ba, w, gq, gk, gdt, gA, gIp, dt_bf16, s);
    default: return launch_bwd_t<128, TIn, TG, false>(fa, ba, w, gq, gk, gdt, gA, gIp, dt_bf16, s);
    }
}

template <int DK, typename TIn, typename TOut>
palimpsa_status launch_bd2(const BdArgs &a, hipStream_t s) {
    constexpr int C = 16;
    const size_t lds = fwd_lds_bytes<DK, C>();
    (void)hipGetLastError();
    if (a.ck) hipLaunchKernelGGL((bd2_fwd_kernel<DK, C, TIn, TOut, true>), dim3(a.nwg), dim3(kThreads), lds, s, a);
    else hipLaunchKernelGGL((bd2_fwd_kernel<DK, C, TIn, TOut>), dim3(a.nwg), dim3(kThreads), lds, s, a);
    return hipGetLastError() == hipSuccess ? PALIMPSA_OK : PALIMPSA_ERR_HIP;
}

template <int DK, typename TIn, typename TOut>
palimpsa_status launch_bd4(const BdArgs &a, hipStream_t s) {
    constexpr int C = 16;
    const size_t lds = fwd_lds_bytes<DK, C>();
    (void)hipGetLastError();
    if (a.ck) hipLaunchKernelGGL((bd4_fwd_kernel<DK, C, TIn, TOut, true>), dim3(a.nwg), dim3(kThreads), lds, s, a);
    else hipLaunchKernelGGL((bd4_fwd_kernel<DK, C, TIn, TOut>), dim3(a.nwg), dim3(kThreads), lds, s, a);
    return hipGetLastError() == hipSuccess ? PALIMPSA_OK : PALIMPSA_ERR_HIP;
}

template <typename TIn, typename TOut>
palimpsa_status launch_bd2_d(const BdArgs &a, int dk, hipStream_t s) {
    switch (dk) {
    case 32: return launch_bd2<32, TIn, TOut>(a, s);
    case 64: return launch_bd2<64, TIn, TOut>(a, s);
    default: return launch_bd2<128, TIn, TOut>(a, s);
    }
}

template <typename TIn, typename TOut>
palimpsa_status launch_bd_d(const BdArgs &a, int dk, int block, hipStream_t s) {
    if (block == 4) return dk == 64 ? launch_bd4<64, TIn, TOut>(a, s) : launch_bd4<128, TIn, TOut>(a, s);
    return launch_bd2_d<TIn, TOut>(a, dk, s);
}

// Block-diagonal backward workspace: the checkpoints (lane states padded to
// float4s), then bwd_kernel's partials in their layouts.
struct BdBwdWs {
    float *ck, *pqk, *ps, *gabh, *gibh, *pI0, *sink;
    size_t bytes;
};
BdBwdWs plan_bd_bwd_ws(void *base, int B, int T, int H, int dk, int dv, int block) {
    const size_t nsb = (size_t)(T + kSB - 1) / kSB, nrb = (size_t)dv / kRowsPerWG;
    const size_t bh = (size_t)B * H, bth = bh * T;
    const size_t kc = (size_t)dk / kLanesPerRow;
    const size_t lane_np = (kc + (block == 2 ? 3 * (kc / 2) : 10 * (kc / 4)) + 3) / 4 * 4;
    size_t off = 0;
    auto take = [&](size_t floats) {
        const size_t o = off;
        off = (off + floats * sizeof(float) + 255) / 256 * 256;
        return o;
    };
    const size_t o_ck = take(bh * nsb * nrb * kThreads * lane_np);
    const size_t o_pqk = take(nrb * bth * 2 * dk), o_ps = take(nrb * bth * 2);
    const size_t o_ga = take(bh), o_gi = take(bh), o_pi = take(bh * nrb);
    // the training forward's discarded checkpoint stores (one workgroup block)
    const size_t o_sink = take((size_t)kThreads * lane_np);
    BdBwdWs w;
    // section pointers only exist for a real base (a size query passes none)
    char *c = (char *)base;
    auto at = [c](size_t o) { return c ? c + o : nullptr; };
    w.ck = (float *)at(o_ck); w.pqk = (float *)at(o_pqk); w.ps = (float *)at(o_ps);
    w.gabh = (float *)at(o_ga); w.gibh = (float *)at(o_gi); w.pI0 = (float *)at(o_pi);
    w.sink = (float *)at(o_sink);
    w.bytes = off;
    return w;
}

template <int DK, int BS, typename TIn, typename TG>
palimpsa_status launch_bd_bwd(const BdBwdArgs &a, const BdBwdWs &w, float *gq, float *gk, float *gdt, float *gA,
                              float *gIp, int dt_bf16, hipStream_t s) {
    (void)hipGetLastError();
    const size_t ck_lds = fwd_lds_bytes<DK, 16>();
    if (a.T > 0 && !a.ck_saved)
        hipLaunchKernelGGL((bd_ckpt_kernel<DK, BS, TIn>), dim3(a.nwg), dim3(kThreads), ck_lds, s, a);
    const size_t lds = (size_t)BwdStage<DK>::kTotal * sizeof(float);
    void (*kern)(BdBwdArgs);
    if constexpr (BS == 2) kern = bd2_bwd_kernel<DK, TIn, TG>;
    else kern = bd4_bwd_kernel<DK, TIn, TG>;
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return PALIMPSA_ERR_HIP;
    hipLaunchKernelGGL(kern, dim3(a.nwg), dim3(kThreads), lds, s, a);
    const size_t bth = (size_t)a.B * a.T * a.H;
    const int nrb = a.dv / kRowsPerWG;
    if (bth > 0) {
        const size_t n4 = bth * (2 * DK / 4);
        hipLaunchKernelGGL(bwd_qk_kernel<DK>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                           (const float *)w.pqk, gq, gk, bth, nrb);
    }
    hipLaunchKernelGGL(bwd_gate_kernel, dim3(a.B * a.H), dim3(256), 0, s, (const float *)w.ps, a.dt, dt_bf16,
                       a.A, a.Ip, 0, 0, gdt, w.gabh, w.gibh, a.B, a.T, a.H, nrb);
    hipLaunchKernelGGL(bwd_head_kernel, dim3((a.H + 63) / 64), dim3(64), 0, s, (const float *)w.gabh,
                       (const float *)w.gibh, (const float *)w.pI0, a.Ip, gA, gIp, a.B, a.H, nrb,
                       a.mu0 ? 0 : 1, 0, 0);
    return hipGetLastError() == hipSuccess ? PALIMPSA_OK : PALIMPSA_ERR_HIP;
}

template <typename TIn, typename TG>
palimpsa_status launch_bd_bwd_d(int dk, int block, const BdBwdArgs &a, const BdBwdWs &w, float *gq, float *gk,
                                float *gdt, float *gA, float *gIp, int dt_bf16, hipStream_t s) {
    if (block == 4)
        return dk == 64 ? launch_bd_bwd<64, 4, TIn, TG>(a, w, gq, gk, gdt, gA, gIp, dt_bf16, s)
                        : launch_bd_bwd<128, 4, TIn, TG>(a, w, gq, gk, gdt, gA, gIp, dt_bf16, s);
    switch (dk) {
    case 32: return launch_bd_bwd<32, 2, TIn, TG>(a, w, gq, gk, gdt, gA, gIp, dt_bf16, s);
    case 64: return launch_bd_bwd<64, 2, TIn, TG>(a, w, gq, gk, gdt, gA, gIp, dt_bf16, s);
    default: return launch_bd_bwd<128, 2, TIn, TG>(a, w, gq, gk, gdt, gA, gIp, dt_bf16, s);
    }
}


}  // namespace

extern "C" {

palimpsa_status palimpsa_fwd_blockdiag(const void *q, const void *k, const void *v, const void *beta,
                                       const void *dt, const float *A, const float *I_prior,
                                       const float *mu0, const float *P0, void *y, float *muT, float *PT,
                                       int B, int T, int H, int dk, int dv, int block,
                                       int in_dtype, int out_dtype, int flags,
                                       void *workspace, size_t workspace_bytes, void *stream) {
    if (!A || !I_prior || (T > 0 && (!q || !k || !v || !beta || !dt || !y)))
        return PALIMPSA_ERR_INVALID_ARG;
    if ((flags & ~PALIMPSA_SAVE_CHECKPOINTS) || ((flags & PALIMPSA_SAVE_CHECKPOINTS) && !workspace))
        return PALIMPSA_ERR_INVALID_ARG;
    if ((mu0 == nullptr) != (P0 == nullptr) || (muT == nullptr) != (PT == nullptr))
        return PALIMPSA_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0 || block <= 0 || !dtype_ok(in_dtype) || !dtype_ok(out_dtype))
        return PALIMPSA_ERR_INVALID_ARG;
    if ((block != 2 && block != 4) || !head_ok(dk) || (block == 4 && dk == 32) || !dv_ok(dv))
        return PALIMPSA_ERR_UNSUPPORTED;
    const bool save = (flags & PALIMPSA_SAVE_CHECKPOINTS) != 0;
    const void *vec_ptrs[] = {q, k, v, beta, P0, PT, save ? workspace : nullptr};
    for (const void *p : vec_ptrs)
        if (p && !aligned_to(p, 16)) return PALIMPSA_ERR_ALIGNMENT;
    const size_t in_sz = in_dtype == PALIMPSA_BF16 ? 2 : 4, out_sz = out_dtype == PALIMPSA_BF16 ? 2 : 4;
    if (!aligned_to(dt, in_sz) || !aligned_to(A, 4) || !aligned_to(I_prior, 4) || (y && !aligned_to(y, out_sz)) ||
        (mu0 && !aligned_to(mu0, 4)) || (muT && !aligned_to(muT, 4)))
        return PALIMPSA_ERR_ALIGNMENT;
    const long long nwg = (long long)B * H * (dv / kRowsPerWG);
    if (nwg > 0x7fffffffLL || (long long)B * T * H * (dk > dv ? dk : dv) > (1LL << 46) ||
        64LL * H * (dk > dv ? dk : dv) >= (1LL << 31))
        return PALIMPSA_ERR_UNSUPPORTED;
    if (save && workspace_bytes < plan_bd_bwd_ws(nullptr, B, T, H, dk, dv, block).bytes)
        return PALIMPSA_ERR_INVALID_ARG;
    if (T == 0 && !muT) return PALIMPSA_OK;
    BdArgs a;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.dt = dt;
    a.A = A; a.Ip = I_prior; a.mu0 = mu0; a.P0 = P0; a.y = y; a.muT = muT; a.PT = PT;
    a.B = B; a.T = T; a.H = H; a.dv = dv;
    a.nwg = (int)nwg; a.xcd_remap = (nwg % 8 == 0) ? 1 : 0;
    a.nsb = (T + kSB - 1) / kSB;
    a.ck = a.ck_sink = nullptr;
    if (save && T > 0) {
        const BdBwdWs w = plan_bd_bwd_ws(workspace, B, T, H, dk, dv, block);
        a.ck = w.ck;
        a.ck_sink = w.sink;
    }
    hipStream_t s = (hipStream_t)stream;
    const bool bf_in = in_dtype == PALIMPSA_BF16, bf_out = out_dtype == PALIMPSA_BF16;
    if (bf_in && bf_out) return launch_bd_d<bf16_t, bf16_t>(a, dk, block, s);
    if (bf_in) return launch_bd_d<bf16_t, float>(a, dk, block, s);
    if (bf_out) return launch_bd_d<float, bf16_t>(a, dk, block, s);
    return launch_bd_d<float, float>(a, dk, block, s);
}

palimpsa_status palimpsa_step_blockdiag(const void *q, const void *k, const void *v, const void *beta,
                                        const void *dt, const float *A, const float *I_prior, float *mu, float *P,
                                        void *y, int B, int H, int dk, int dv, int block,
                                        int in_dtype, int out_dtype, void *stream) {
    if (!q || !k || !v || !beta || !dt || !A || !I_prior || !mu || !P || !y)
        return PALIMPSA_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || dk <= 0 || dv <= 0 || block <= 0 || !dtype_ok(in_dtype) || !dtype_ok(out_dtype))
        return PALIMPSA_ERR_INVALID_ARG;
    if ((block != 2 && block != 4) || !head_ok(dk) || (block == 4 && dk == 32) || !dv_ok(dv))
        return PALIMPSA_ERR_UNSUPPORTED;
    if (!aligned_to(mu, 16) || !aligned_to(P, 16))
        return PALIMPSA_ERR_ALIGNMENT;
    const size_t in_sz = in_dtype == PALIMPSA_BF16 ? 2 : 4, out_sz = out_dtype == PALIMPSA_BF16 ? 2 : 4;
    const void *in_ptrs[] = {q, k, v, beta, dt};
    for (const void *p : in_ptrs)
        if (!aligned_to(p, in_sz)) return PALIMPSA_ERR_ALIGNMENT;
    if (!aligned_to(A, 4) || !aligned_to(I_prior, 4) || !aligned_to(y, out_sz)) return PALIMPSA_ERR_ALIGNMENT;
    const long long rows = (long long)B * H * dv;
    if (rows * dk > (1LL << 46))
        return PALIMPSA_ERR_UNSUPPORTED;
    Bd2StepArgs a;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.dt = dt;
    a.A = A; a.Ip = I_prior; a.mu = mu; a.P = P; a.y = y;
    a.H = H; a.dv = dv; a.rows = rows;
    const int rows_per_block = kStepThreads / (dk / 4);
    const long long blocks = (rows + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7fffffffLL) return PALIMPSA_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    const bool bf_in = in_dtype == PALIMPSA_BF16, bf_out = out_dtype == PALIMPSA_BF16;
    const bool i32 = rows <= 0xffffffffLL;
    (void)hipGetLastError();
#define PALIMPSA_BD2_STEP_LAUNCH(DK_, TI, TO)                                                                   \
    do {                                                                                                        \
        if (block == 4 && i32)                                                                                  \
            hipLaunchKernelGGL((bd4_step_kernel<DK_ == 32 ? 64 : DK_, TI, TO, true>), dim3((unsigned)blocks),   \
                               dim3(kStepThreads), 0, s, a);                                                    \
        else if (block == 4)                                                                                    \
            hipLaunchKernelGGL((bd4_step_kernel<DK_ == 32 ? 64 : DK_, TI, TO>), dim3((unsigned)blocks),         \
                               dim3(kStepThreads), 0, s, a);                                                    \
        else if (i32)                                                                                           \
            hipLaunchKernelGGL((bd2_step_kernel<DK_, TI, TO, true>), dim3((unsigned)blocks), dim3(kStepThreads), \
                               0, s, a);                                                                        \
        else                                                                                                    \
            hipLaunchKernelGGL((bd2_step_kernel<DK_, TI, TO>), dim3((unsigned)blocks), dim3(kStepThreads), 0, s, a); \
    } while (0)
#define PALIMPSA_BD2_STEP_TYPES(DK_)                                          \
    do {                                                                      \
        if (bf_in && bf_out) PALIMPSA_BD2_STEP_LAUNCH(DK_, bf16_t, bf16_t);   \
        else if (bf_in) PALIMPSA_BD2_STEP_LAUNCH(DK_, bf16_t, float);         \
        else if (bf_out) PALIMPSA_BD2_STEP_LAUNCH(DK_, float, bf16_t);        \
        else PALIMPSA_BD2_STEP_LAUNCH(DK_, float, float);                     \
    } while (0)
    switch (dk) {
    case 32: PALIMPSA_BD2_STEP_TYPES(32); break;
    case 64: PALIMPSA_BD2_STEP_TYPES(64); break;
    default: PALIMPSA_BD2_STEP_TYPES(128); break;
    }
#undef PALIMPSA_BD2_STEP_TYPES
#undef PALIMPSA_BD2_STEP_LAUNCH
    return hipGetLastError() == hipSuccess ? PALIMPSA_OK : PALIMPSA_ERR_HIP;
}

size_t palimpsa_bwd_blockdiag_workspace_size(int B, int T, int H, int dk, int dv, int block) {
    if (B <= 0 || H <= 0 || T < 0 || (block != 2 && block != 4) || !head_ok(dk) || (block == 4 && dk == 32) ||
        !dv_ok(dv))
        return 0;
    return plan_bd_bwd_ws(nullptr, B, T, H, dk, dv, block).bytes;
}

palimpsa_status palimpsa_bwd_blockdiag(const void *q, const void *k, const void *v, const void *beta,
                                       const void *dt, const float *A, const float *I_prior,
                                       const float *mu0, const float *P0,
                                       const void *gy, const float *gmuT, const float *gPT,
                                       float *gq, float *gk, float *gv, float *gbeta, float *gdt,
                                       float *gA, float *gIp, float *gmu0, float *gP0,
                                       int B, int T, int H, int dk, int dv, int block,
                                       int in_dtype, int gy_dtype, int flags,
                                       void *workspace, size_t workspace_bytes, void *stream) {
    if (!A || !I_prior || !gA || !gIp || !workspace || (flags & ~PALIMPSA_CHECKPOINTS_SAVED))
        return PALIMPSA_ERR_INVALID_ARG;
    if (T > 0 && (!q || !k || !v || !beta || !dt || !gy || !gq || !gk || !gv || !gbeta || !gdt))
        return PALIMPSA_ERR_INVALID_ARG;
    if ((mu0 == nullptr) != (P0 == nullptr))
        return PALIMPSA_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0 || block <= 0 || !dtype_ok(in_dtype) ||
        !dtype_ok(gy_dtype))
        return PALIMPSA_ERR_INVALID_ARG;
    if ((block != 2 && block != 4) || !head_ok(dk) || (block == 4 && dk == 32) || !dv_ok(dv))
        return PALIMPSA_ERR_UNSUPPORTED;
    const void *vec_ptrs[] = {q, k, v, beta, gy, P0, gPT, gP0, gq, gk, workspace};
    for (const void *p : vec_ptrs)
        if (p && !aligned_to(p, 16)) return PALIMPSA_ERR_ALIGNMENT;
    const size_t in_sz = in_dtype == PALIMPSA_BF16 ? 2 : 4;
    const void *f32_ptrs[] = {A, I_prior, gA, gIp, gv, gbeta, gdt, mu0, gmuT, gmu0};
    for (const void *p : f32_ptrs)
        if (p && !aligned_to(p, 4)) return PALIMPSA_ERR_ALIGNMENT;
    if (dt && !aligned_to(dt, in_sz)) return PALIMPSA_ERR_ALIGNMENT;
    const long long nwg = (long long)B * H * (dv / kRowsPerWG);
    if (nwg > 0x7fffffffLL || (long long)B * T * H * (dk > dv ? dk : dv) > (1LL << 46) ||
        64LL * H * (dk > dv ? dk : dv) >= (1LL << 31) || (long long)B * H * 2 > 0x7fffffffLL)
        return PALIMPSA_ERR_UNSUPPORTED;
    const BdBwdWs w = plan_bd_bwd_ws(workspace, B, T, H, dk, dv, block);
    if (workspace_bytes < w.bytes) return PALIMPSA_ERR_INVALID_ARG;

    BdBwdArgs a = {};
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.dt = dt; a.gy = gy;
    a.A = A; a.Ip = I_prior; a.mu0 = mu0; a.P0 = P0; a.gmuT = gmuT; a.gPT = gPT;
    a.gv = gv; a.gbeta = gbeta; a.gmu0 = gmu0; a.gP0 = gP0;
    a.ck = w.ck; a.pqk = w.pqk; a.ps = w.ps; a.pI0 = w.pI0;
    a.B = B; a.T = T; a.H = H; a.dv = dv; a.nsb = (T + kSB - 1) / kSB;
    a.ck_saved = (flags & PALIMPSA_CHECKPOINTS_SAVED) ? 1 : 0;
    a.nwg = (int)nwg; a.xcd_remap = (nwg % 8 == 0) ? 1 : 0;
    hipStream_t s = (hipStream_t)stream;
    const bool bf_in = in_dtype == PALIMPSA_BF16, bf_gy = gy_dtype == PALIMPSA_BF16;
    const int dtb = bf_in ? 1 : 0;
    if (bf_in && bf_gy) return launch_bd_bwd_d<bf16_t, bf16_t>(dk, block, a, w, gq, gk, gdt, gA, gIp, dtb, s);
    if (bf_in) return launch_bd_bwd_d<bf16_t, float>(dk, block, a, w, gq, gk, gdt, gA, gIp, dtb, s);
    if (bf_gy) return launch_bd_bwd_d<float, bf16_t>(dk, block, a, w, gq, gk, gdt, gA, gIp, dtb, s);
    return launch_bd_bwd_d<float, float>(dk, block, a, w, gq, gk, gdt, gA, gIp, dtb, s);
}

size_t palimpsa_bwd_workspace_size(int B, int T, int H, int dk, int dv, int flags) {
    if (B <= 0 || H <= 0 || T < 0 || !head_ok(dk) || !dv_ok(dv) || (flags & ~(kFlagsFwd | kFlagsBwd))) return 0;
    return plan_bwd_ws(nullptr, B, T, H, dk, dv, (flags & PALIMPSA_PRIOR_PER_ENTRY) != 0).bytes;
}

palimpsa_status palimpsa_bwd(const void *q, const void *k, const void *v, const void *beta, const void *dt,
                             const float *A, const float *I_prior, const float *mu0, const float *I0,
                             const void *gy, const float *gmuT, const float *gIT,
                             float *gq, float *gk, float *gv, float *gbeta, float *gdt,
                             float *gA, float *gIp, float *gmu0, float *gI0,
                             int B, int T, int H, int dk, int dv,
                             int in_dtype, int gy_dtype, int flags,
                             void *workspace, size_t workspace_bytes, void *stream) {
    if (!A || !I_prior || !gA || !gIp || !workspace || (flags & ~kFlagsBwd))
        return PALIMPSA_ERR_INVALID_ARG;
    if (T > 0 && (!q || !k || !v || !beta || !dt || !gy || !gq || !gk || !gv || !gbeta || !gdt))
        return PALIMPSA_ERR_INVALID_ARG;
    if ((mu0 == nullptr) != (I0 == nullptr))
        return PALIMPSA_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0 || !dtype_ok(in_dtype) || !dtype_ok(gy_dtype))
        return PALIMPSA_ERR_INVALID_ARG;
    if (!head_ok(dk) || !dv_ok(dv))
        return PALIMPSA_ERR_UNSUPPORTED;
    const bool ipe = (flags & PALIMPSA_PRIOR_PER_ENTRY) != 0;
    const void *vec_ptrs[] = {q, k, v, beta, gy, mu0, I0, gmuT, gIT, gq, gk, gmu0, gI0, workspace,
                              ipe ? (const void *)I_prior : nullptr, ipe ? (const void *)gIp : nullptr};
    for (const void *p : vec_ptrs)
        if (p && !aligned_to(p, 16)) return PALIMPSA_ERR_ALIGNMENT;
    const size_t in_sz = in_dtype == PALIMPSA_BF16 ? 2 : 4;
    const void *f32_ptrs[] = {A, I_prior, gA, gIp, gv, gbeta, gdt};
    for (const void *p : f32_ptrs)
        if (p && !aligned_to(p, 4)) return PALIMPSA_ERR_ALIGNMENT;
    if (dt && !aligned_to(dt, in_sz)) return PALIMPSA_ERR_ALIGNMENT;
    const long long nwg = (long long)B * H * (dv / kRowsPerWG);
    if (nwg > 0x7fffffffLL || (long long)B * T * H * (dk > dv ? dk : dv) > (1LL << 46) ||
        64LL * H * (dk > dv ? dk : dv) >= (1LL << 31) || (long long)B * H * 2 > 0x7fffffffLL)
        return PALIMPSA_ERR_UNSUPPORTED;
    const BwdWs w = plan_bwd_ws(workspace, B, T, H, dk, dv, ipe);
    if (workspace_bytes < w.bytes) return PALIMPSA_ERR_INVALID_ARG;

    FwdArgs fa = {};
    fa.q = q; fa.k = k; fa.v = v; fa.beta = beta; fa.dt = dt;
    fa.A = A; fa.Ip = I_prior; fa.mu0 = mu0; fa.I0 = I0;
    fa.B = B; fa.T = T; fa.H = H; fa.dv = dv;
    fa.nwg = (int)nwg; fa.xcd_remap = (nwg % 8 == 0) ? 1 : 0; fa.nwg_seg = (int)nwg;
    fa.seg_len = T > 0 ? T : 1; fa.nseg = 1;
    fa.ck = (flags & PALIMPSA_CHECKPOINTS_SAVED) ? nullptr : w.ck;
    fa.nck = (T + kCkI - 1) / kCkI;
    fa.vstar = (flags & PALIMPSA_VSTAR) ? 1 : 0;

    BwdArgs ba = {};
    ba.q = q; ba.k = k; ba.v = v; ba.beta = beta; ba.dt = dt; ba.gy = gy;
    ba.A = A; ba.Ip = I_prior; ba.mu0 = mu0; ba.I0 = I0; ba.gmuT = gmuT; ba.gIT = gIT;
    ba.gv = gv; ba.gbeta = gbeta; ba.gmu0 = gmu0; ba.gI0 = gI0;
    ba.ck = w.ck; ba.pqk = w.pqk; ba.ps = w.ps; ba.pI0 = w.pI0; ba.pip = w.pip;
    ba.vstar = fa.vstar;
    ba.B = B; ba.T = T; ba.H = H; ba.dv = dv; ba.nsb = (T + kSB - 1) / kSB; ba.nck = fa.nck;
    ba.nwg = (int)nwg; ba.xcd_remap = fa.xcd_remap;

    hipStream_t s = (hipStream_t)stream;
    const bool bf_in = in_dtype == PALIMPSA_BF16, bf_gy = gy_dtype == PALIMPSA_BF16;
    const int dtb = bf_in ? 1 : 0;
    if (bf_in && bf_gy) return launch_bwd_d<bf16_t, bf16_t>(dk, ipe, fa, ba, w, gq, gk, gdt, gA, gIp, dtb, s);
    if (bf_in) return launch_bwd_d<bf16_t, float>(dk, ipe, fa, ba, w, gq, gk, gdt, gA, gIp, dtb, s);
    if (bf_gy) return launch_bwd_d<float, bf16_t>(dk, ipe, fa, ba, w, gq, gk, gdt, gA, gIp, dtb, s);
    return launch_bwd_d<float, float>(dk, ipe, fa, ba, w, gq, gk, gdt, gA, gIp, dtb, s);
}

palimpsa_status palimpsa_bwd_frozen(const void *q, const void *k, const void *v, const void *beta,
                                    const void *dt, const float *A, const float *I_prior, const float *mu0,
                                    const void *gy, const float *gmuT,
                                    float *gq, float *gk, float *gv, float *gbeta, float *gdt,
                                    float *gA, float *gIp, float *gmu0,
                                    int B, int T, int H, int dk, int dv,
                                    int in_dtype, int gy_dtype,
                                    void *workspace, size_t workspace_bytes, void *stream) {
    if (!A || !I_prior || !gA || !gIp || !workspace)
        return PALIMPSA_ERR_INVALID_ARG;
    if (T > 0 && (!q || !k || !v || !dt || !gy || !gq || !gk || !gv || !gdt || (beta && !gbeta)))
        return PALIMPSA_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0 || !dtype_ok(in_dtype) || !dtype_ok(gy_dtype))
        return PALIMPSA_ERR_INVALID_ARG;
    if (!head_ok(dk) || !dv_ok(dv))
        return PALIMPSA_ERR_UNSUPPORTED;
    const void *vec_ptrs[] = {q, k, v, beta, gy, mu0, gmuT, gq, gk, gmu0, workspace};
    for (const void *p : vec_ptrs)
        if (p && !aligned_to(p, 16)) return PALIMPSA_ERR_ALIGNMENT;
    const size_t in_sz = in_dtype == PALIMPSA_BF16 ? 2 : 4;
    const void *f32_ptrs[] = {A, I_prior, gA, gIp, gv, gbeta, gdt};
    for (const void *p : f32_ptrs)
        if (p && !aligned_to(p, 4)) return PALIMPSA_ERR_ALIGNMENT;
    if (dt && !aligned_to(dt, in_sz)) return PALIMPSA_ERR_ALIGNMENT;
    const long long nwg = (long long)B * H * (dv / kRowsPerWG);
    if (nwg > 0x7fffffffLL || (long long)B * T * H * (dk > dv ? dk : dv) > (1LL << 46) ||
        64LL * H * (dk > dv ? dk : dv) >= (1LL << 31) || (long long)B * H * 2 > 0x7fffffffLL)
        return PALIMPSA_ERR_UNSUPPORTED;
    const BwdWs w = plan_bwd_ws(workspace, B, T, H, dk, dv, false);
    if (workspace_bytes < w.bytes) return PALIMPSA_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    if (in_dtype == PALIMPSA_BF16 && (dk == 64 || dk == 128) && (dv == 64 || dv == 128 || dv == 256)) {
        // chunked form on the matrix cores
        const FzbWs fw = plan_fzb_ws(workspace, B, T, H, dk, dv);
        if (fw.bytes > w.bytes) return PALIMPSA_ERR_INVALID_ARG;
        FzbArgs fa;
        fa.q = (const bf16_t *)q; fa.k = (const bf16_t *)k; fa.v = (const bf16_t *)v;
        fa.beta = (const bf16_t *)beta; fa.dt = (const bf16_t *)dt; fa.gy = gy;
        fa.A = A; fa.Ip = I_prior; fa.mu0 = mu0; fa.gmuT = gmuT;
        fa.gq = gq; fa.gk = gk; fa.gv = gv; fa.gbeta = beta ? gbeta : nullptr; fa.gdt = gdt;
        fa.gA = gA; fa.gIp = gIp; fa.gmu0 = gmu0;
        fa.sT = fw.sT; fa.ge = fw.ge; fa.gT = fw.gT;
        fa.pA = fw.pA; fa.pI = fw.pI;
        fa.B = B; fa.T = T; fa.H = H; fa.nc = (T + kFbC - 1) / kFbC;
        fa.vec_g = aligned_to(gv, 16) && (!beta || aligned_to(gbeta, 16));
        return gy_dtype == PALIMPSA_BF16 ? launch_fzb_d<bf16_t>(dk, dv, fa, s) : launch_fzb_d<float>(dk, dv, fa, s);
    }
    // without beta the v tensor is the write itself; the beta pointer is then
    // pointed at v so that every staged load stays valid (the frozen walk
    // never reads it)
    const void *bsrc = beta ? beta : v;

    FwdArgs fa = {};
    fa.q = q; fa.k = k; fa.v = v; fa.beta = bsrc; fa.dt = dt;
    fa.A = A; fa.Ip = I_prior; fa.mu0 = mu0; fa.I0 = nullptr;
    fa.B = B; fa.T = T; fa.H = H; fa.dv = dv;
    fa.nwg = (int)nwg; fa.xcd_remap = (nwg % 8 == 0) ? 1 : 0; fa.nwg_seg = (int)nwg;
    fa.seg_len = T > 0 ? T : 1; fa.nseg = 1;
    fa.ck = w.ck; fa.nck = (T + kCkI - 1) / kCkI;
    fa.vstar = beta ? 0 : 1;
    fa.frozen = 1;

    BwdArgs ba = {};
    ba.q = q; ba.k = k; ba.v = v; ba.beta = bsrc; ba.dt = dt; ba.gy = gy;
    ba.A = A; ba.Ip = I_prior; ba.mu0 = mu0; ba.I0 = nullptr; ba.gmuT = gmuT; ba.gIT = nullptr;
    ba.gv = gv; ba.gbeta = beta ? gbeta : nullptr; ba.gmu0 = gmu0; ba.gI0 = nullptr;
    ba.ck = w.ck; ba.pqk = w.pqk; ba.ps = w.ps; ba.pI0 = w.pI0; ba.pip = nullptr;
    ba.vstar = fa.vstar;
    ba.B = B; ba.T = T; ba.H = H; ba.dv = dv; ba.nsb = (T + kSB - 1) / kSB; ba.nck = fa.nck;
    ba.nwg = (int)nwg; ba.xcd_remap = fa.xcd_remap;

    const bool bf_in = in_dtype == PALIMPSA_BF16, bf_gy = gy_dtype == PALIMPSA_BF16;
    const int dtb = bf_in ? 1 : 0;
    if (bf_in && bf_gy) return launch_bwd_fz_d<bf16_t, bf16_t>(dk, fa, ba, w, gq, gk, gdt, gA, gIp, dtb, s);
    if (bf_in) return launch_bwd_fz_d<bf16_t, float>(dk, fa, ba, w, gq, gk, gdt, gA, gIp, dtb, s);
    if (bf_gy) return launch_bwd_fz_d<float, bf16_t>(dk, fa, ba, w, gq, gk, gdt, gA, gIp, dtb, s);
    return launch_bwd_fz_d<float, float>(dk, fa, ba, w, gq, gk, gdt, gA, gIp, dtb, s);
}

palimpsa_status palimpsa_fwd_frozen(const void *q, const void *k, const void *v,
                                    const void *beta, const void *dt,
                                    const float *A, const float *I_prior, const float *mu0,
                                    void *y, float *muT, int B, int T, int H, int dk, int dv,
                                    int in_dtype, int out_dtype,
                                    void *stream) {
    if (!A || !I_prior || (T > 0 && (!q || !k || !v || !dt || !y)))
        return PALIMPSA_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0)
        return PALIMPSA_ERR_INVALID_ARG;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
        return PALIMPSA_ERR_INVALID_ARG;
    if (in_dtype != PALIMPSA_BF16 || (dk != 64 && dk != 128) || !dv_ok(dv) || dv % kFzRows != 0)
        return PALIMPSA_ERR_UNSUPPORTED;
    const void *vec_ptrs[] = {q, k, v, beta, mu0, muT, y};
    for (const void *p : vec_ptrs)
        if (p && !aligned_to(p, 16)) return PALIMPSA_ERR_ALIGNMENT;
    if (!aligned_to(dt, 2) || !aligned_to(A, 4) || !aligned_to(I_prior, 4))
        return PALIMPSA_ERR_ALIGNMENT;
    if ((long long)B * H * (dv / kFzRows) > 0x7fffffffLL || (long long)B * T * H * (dk > dv ? dk : dv) > (1LL << 46))
        return PALIMPSA_ERR_UNSUPPORTED;
    FrozenArgs a;
    a.q = (const bf16_t *)q; a.k = (const bf16_t *)k; a.v = (const bf16_t *)v;
    a.beta = (const bf16_t *)beta; a.dt = (const bf16_t *)dt;
    a.A = A; a.Ip = I_prior; a.mu0 = mu0; a.y = y; a.muT = muT;
    a.B = B; a.T = T; a.H = H; a.dv = dv;
    a.y_bf16 = out_dtype == PALIMPSA_BF16;
    if (T == 0 && !muT) return PALIMPSA_OK;
    hipStream_t s = (hipStream_t)stream;
    return dk == 64 ? launch_frozen<64>(a, s) : launch_frozen<128>(a, s);
}


size_t palimpsa_fwd_workspace_size(int B, int T, int H, int dk, int dv, int segments) {
    if (B <= 0 || H <= 0 || T < 0 || !fwd_dk_ok(dk) || !fwd_dv_ok(dv) || segments < 0) return 0;
    if (dk > 256) {
        WideRowsPlan p;
        return plan_wide_rows(B, T, H, dk, dv, device_cus(), &p) ? p.bytes : 0;
    }
    return plan_segments(B, T, H, dk, dv, segments, device_cus()).ws_bytes;
}

}  // extern "C"

namespace {

// The chunked forward behind both entry points.  noalloc: the caller passes
// no workspace; a split runs in this device's fixed scratch array instead,
// and a call whose split would need more than that array holds is refused.
palimpsa_status fwd_chunked_impl(const void *q, const void *k, const void *v,
                                 const void *beta, const void *dt,
                                 const float *A, const float *I_prior,
                                 const float *mu0, const float *I0,
                                 void *y, float *muT, float *IT,
                                 int B, int T, int H, int dk, int dv, int chunk, int segments,
                                 int in_dtype, int out_dtype, int flags,
                                 void *workspace, size_t workspace_bytes, void *stream, bool noalloc) {
    if (!A || !I_prior || (T > 0 && (!q || !k || !v || !beta || !dt || !y)) || (flags & ~kFlagsFwd))
        return PALIMPSA_ERR_INVALID_ARG;
    if (noalloc && (flags & PALIMPSA_SAVE_CHECKPOINTS))   // that workspace is a backward's, gigabytes
        return PALIMPSA_ERR_INVALID_ARG;
    if ((mu0 == nullptr) != (I0 == nullptr) || (muT == nullptr) != (IT == nullptr))
        return PALIMPSA_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0)
        return PALIMPSA_ERR_INVALID_ARG;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
        return PALIMPSA_ERR_INVALID_ARG;
    if (chunk != 0 && chunk != 8 && chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128)
        return PALIMPSA_ERR_INVALID_ARG;
    if (segments < 0 || segments > 64 || (workspace_bytes > 0 && !workspace))
        return PALIMPSA_ERR_INVALID_ARG;
    if (!fwd_dk_ok(dk) || !fwd_dv_ok(dv))
        return PALIMPSA_ERR_UNSUPPORTED;
    // heads wider than 128 keys: per-head prior, v as given, one pass (no time split)
    if (dk > 128 && (flags != 0 || (dv % 16) != 0 || (dk == 256 && dv > 1024)))
        return PALIMPSA_ERR_UNSUPPORTED;
    // training forward: one pass at chunk 16 within the backward's sizes
    const bool save_ck = (flags & PALIMPSA_SAVE_CHECKPOINTS) != 0;
    if (save_ck) {
        if (!head_ok(dk) || !dv_ok(dv) || segments > 1 || (chunk != 0 && chunk != 16))
            return PALIMPSA_ERR_UNSUPPORTED;
        if (!workspace) return PALIMPSA_ERR_INVALID_ARG;
    }
    if (dk > 256) segments = segments >= 2 ? -1 : 1;
    if (segments < 0) return PALIMPSA_ERR_UNSUPPORTED;
    const bool ipe = (flags & PALIMPSA_PRIOR_PER_ENTRY) != 0;
    // 128-bit accesses: q, k, v, beta, the state arrays (and a per-entry prior) and
    // the workspace; element-wise: the rest
    const void *vec_ptrs[] = {q, k, v, beta, mu0, I0, muT, IT, workspace, ipe ? (const void *)I_prior : nullptr};
    for (const void *p : vec_ptrs)
        if (p && !aligned_to(p, 16)) return PALIMPSA_ERR_ALIGNMENT;
    const size_t in_sz = in_dtype == PALIMPSA_BF16 ? 2 : 4, out_sz = out_dtype == PALIMPSA_BF16 ? 2 : 4;
    if (!aligned_to(dt, in_sz) || !aligned_to(A, 4) || !aligned_to(I_prior, 4) || (y && !aligned_to(y, out_sz)))
        return PALIMPSA_ERR_ALIGNMENT;
    const long long nwg = (long long)B * H * (dv / kRowsPerWG);
    // per-chunk staging offsets are 32-bit: 64 tokens x H x d must stay below 2^31
    if (nwg > 0x7fffffffLL || (long long)B * T * H * (dk > dv ? dk : dv) > (1LL << 46) ||
        64LL * H * (dk > dv ? dk : dv) >= (1LL << 31))
        return PALIMPSA_ERR_UNSUPPORTED;

    FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.dt = dt;
    a.A = A; a.Ip = I_prior; a.mu0 = mu0; a.I0 = I0;
    a.y = y; a.muT = muT; a.IT = IT;
    a.B = B; a.T = T; a.H = H; a.dv = dv;
    a.nwg = (int)nwg;
    a.xcd_remap = (nwg % 8 == 0) ? 1 : 0;
    a.nwg_seg = (int)nwg;
    a.vstar = (flags & PALIMPSA_VSTAR) ? 1 : 0;
    a.ck = nullptr; a.nck = 0; a.frozen = 0;
    if (save_ck) {
        if ((long long)B * H * 2 > 0x7fffffffLL) return PALIMPSA_ERR_UNSUPPORTED;
        const BwdWs w = plan_bwd_ws(workspace, B, T, H, dk, dv, ipe);
        if (workspace_bytes < w.bytes) return PALIMPSA_ERR_INVALID_ARG;
        if (T == 0 && !muT) return PALIMPSA_OK;
        a.ck = w.ck; a.nck = (T + kCkI - 1) / kCkI;
        a.nseg = 1; a.seg_len = T > 0 ? T : 1; a.ws = nullptr;
        hipStream_t s = (hipStream_t)stream;
        const bool bf_in = in_dtype == PALIMPSA_BF16, bf_out = out_dtype == PALIMPSA_BF16;
        if (bf_in && bf_out) return launch_fwd_ckpt<bf16_t, bf16_t>(a, dk, ipe, s);
        if (bf_in) return launch_fwd_ckpt<bf16_t, float>(a, dk, ipe, s);
        if (bf_out) return launch_fwd_ckpt<float, bf16_t>(a, dk, ipe, s);
        return launch_fwd_ckpt<float, float>(a, dk, ipe, s);
    }

    if (T == 0 && !muT) return PALIMPSA_OK;   // nothing to compute or write
    hipStream_t s = (hipStream_t)stream;
    const bool bf_in = in_dtype == PALIMPSA_BF16, bf_out = out_dtype == PALIMPSA_BF16;
    WideRowsPlan wp;
    if (!noalloc && workspace && plan_wide_rows(B, T, H, dk, dv, device_cus(), &wp) && workspace_bytes >= wp.bytes) {
        if (bf_in && bf_out) return launch_wide_rows_d<bf16_t, bf16_t>(a, dk, wp, workspace, s);
        if (bf_in) return launch_wide_rows_d<bf16_t, float>(a, dk, wp, workspace, s);
        if (bf_out) return launch_wide_rows_d<float, bf16_t>(a, dk, wp, workspace, s);
        return launch_wide_rows_d<float, float>(a, dk, wp, workspace, s);
    }
    SegPlan plan = plan_segments(B, T, H, dk, dv, segments, device_cus());
    if (noalloc && plan.nseg > 1) {
        if (plan.ws_bytes > kNoAllocScratchBytes) return PALIMPSA_ERR_SCRATCH_LIMIT;
        palimpsa_status st;
        workspace = device_scratch(&st);
        if (st != PALIMPSA_OK) return st;
        workspace_bytes = kNoAllocScratchBytes;
    }
    if (plan.nseg > 1 && (!workspace || workspace_bytes < plan.ws_bytes)) {
        if (segments >= 2) return PALIMPSA_ERR_INVALID_ARG;     // a split was asked for explicitly
        plan = plan_segments(B, T, H, dk, dv, 1, 256);          // auto: run unsplit
    }
    if (nwg * plan.nseg * 4 > 0x7fffffffLL) return PALIMPSA_ERR_UNSUPPORTED;   // (summary: up to 4 column slices)
    a.nseg = plan.nseg;
    a.seg_len = plan.seg_len;
    a.ws = (float *)workspace;
    const int C = pick_chunk(chunk, dk, nwg * plan.nseg, device_lds_max());
    if (bf_in && bf_out) return launch_fwd_d<bf16_t, bf16_t>(a, dk, C, ipe, s);
    if (bf_in) return launch_fwd_d<bf16_t, float>(a, dk, C, ipe, s);
    if (bf_out) return launch_fwd_d<float, bf16_t>(a, dk, C, ipe, s);
    return launch_fwd_d<float, float>(a, dk, C, ipe, s);
}

}  // namespace

extern "C" {

palimpsa_status palimpsa_fwd_chunked(const void *q, const void *k, const void *v,
                                     const void *beta, const void *dt,
                                     const float *A, const float *I_prior,
                                     const float *mu0, const float *I0,
                                     void *y, float *muT, float *IT,
                                     int B, int T, int H, int dk, int dv, int chunk, int segments,
                                     int in_dtype, int out_dtype, int flags,
                                     void *workspace, size_t workspace_bytes, void *stream) {
    return fwd_chunked_impl(q, k, v, beta, dt, A, I_prior, mu0, I0, y, muT, IT, B, T, H, dk, dv, chunk,
                            segments, in_dtype, out_dtype, flags, workspace, workspace_bytes, stream, false);
}

palimpsa_status palimpsa_fwd_chunked_noalloc(const void *q, const void *k, const void *v,
                                             const void *beta, const void *dt,
                                             const float *A, const float *I_prior,
                                             const float *mu0, const float *I0,
                                             void *y, float *muT, float *IT,
                                             int B, int T, int H, int dk, int dv, int chunk, int segments,
                                             int in_dtype, int out_dtype, int flags,
                                             void *stream) {
    return fwd_chunked_impl(q, k, v, beta, dt, A, I_prior, mu0, I0, y, muT, IT, B, T, H, dk, dv, chunk,
                            segments, in_dtype, out_dtype, flags, nullptr, 0, stream, true);
}

size_t palimpsa_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

palimpsa_status palimpsa_step(const void *q, const void *k, const void *v,
                              const void *beta, const void *dt,
                              const float *A, const float *I_prior,
                              float *mu, float *I, void *y,
                              int B, int H, int dk, int dv,
                              int in_dtype, int out_dtype, int flags,
                              void *stream) {
    if (!q || !k || !v || !beta || !dt || !A || !I_prior || !mu || !I || !y || (flags & ~kFlagsOptions))
        return PALIMPSA_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || dk <= 0 || dv <= 0)
        return PALIMPSA_ERR_INVALID_ARG;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
        return PALIMPSA_ERR_INVALID_ARG;
    if (!fwd_dk_ok(dk) || !fwd_dv_ok(dv))
        return PALIMPSA_ERR_UNSUPPORTED;
    const bool ipe = (flags & PALIMPSA_PRIOR_PER_ENTRY) != 0;
    // 128-bit accesses: the state (and a per-entry prior); element-wise: the rest
    if (!aligned_to(mu, 16) || !aligned_to(I, 16) || (ipe && !aligned_to(I_prior, 16)))
        return PALIMPSA_ERR_ALIGNMENT;
    const size_t in_sz = in_dtype == PALIMPSA_BF16 ? 2 : 4, out_sz = out_dtype == PALIMPSA_BF16 ? 2 : 4;
    const void *in_ptrs[] = {q, k, v, beta, dt};
    for (const void *p : in_ptrs)
        if (!aligned_to(p, in_sz)) return PALIMPSA_ERR_ALIGNMENT;
    if (!aligned_to(A, 4) || !aligned_to(I_prior, 4) || !aligned_to(y, out_sz)) return PALIMPSA_ERR_ALIGNMENT;
    const long long rows = (long long)B * H * dv;
    if (rows * dk > (1LL << 46))
        return PALIMPSA_ERR_UNSUPPORTED;

    StepArgs a;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.dt = dt;
    a.A = A; a.Ip = I_prior; a.mu = mu; a.I = I; a.y = y;
    a.B = B; a.H = H; a.dv = dv; a.rows = rows;
    a.vstar = (flags & PALIMPSA_VSTAR) ? 1 : 0;
    a.ipe = ipe ? 1 : 0;
    const int rows_per_block = kStepThreads / (dk / 4 < 32 ? dk / 4 : 32);
    const long long blocks = (rows + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7fffffffLL) return PALIMPSA_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    const bool bf_in = in_dtype == PALIMPSA_BF16, bf_out = out_dtype == PALIMPSA_BF16;
    (void)hipGetLastError();
#define PALIMPSA_STEP_LAUNCH(DK_, TI, TO) \
    hipLaunchKernelGGL((step_kernel<DK_, TI, TO>), dim3((unsigned)blocks), dim3(kStepThreads), 0, s, a)
#define PALIMPSA_STEP_TYPES(DK_)                                              \
    do {                                                                      \
        if (bf_in && bf_out) PALIMPSA_STEP_LAUNCH(DK_, bf16_t, bf16_t);       \
        else if (bf_in) PALIMPSA_STEP_LAUNCH(DK_, bf16_t, float);             \
        else if (bf_out) PALIMPSA_STEP_LAUNCH(DK_, float, bf16_t);            \
        else PALIMPSA_STEP_LAUNCH(DK_, float, float);                         \
    } while (0)
    switch (dk) {
    case 32: PALIMPSA_STEP_TYPES(32); break;
    case 64: PALIMPSA_STEP_TYPES(64); break;
    case 256: PALIMPSA_STEP_TYPES(256); break;
    case 512: PALIMPSA_STEP_TYPES(512); break;
    case 1024: PALIMPSA_STEP_TYPES(1024); break;
    case 2048: PALIMPSA_STEP_TYPES(2048); break;
    default: PALIMPSA_STEP_TYPES(128); break;
    }
#undef PALIMPSA_STEP_TYPES
#undef PALIMPSA_STEP_LAUNCH
    return hipGetLastError() == hipSuccess ? PALIMPSA_OK : PALIMPSA_ERR_HIP;
}

const char *palimpsa_status_string(int status) {
    switch (status) {
    case PALIMPSA_OK: return "ok";
    case PALIMPSA_ERR_INVALID_ARG: return "invalid argument (null pointer, size or enum)";
    case PALIMPSA_ERR_UNSUPPORTED: return "unsupported configuration (head size must be 32, 64 or 128)";
    case PALIMPSA_ERR_ALIGNMENT: return "tensor pointer misaligned (see palimpsa.h)";
    case PALIMPSA_ERR_HIP: return "HIP runtime error at launch";
    case PALIMPSA_ERR_SCRATCH_LIMIT:
        return "the call needs more scratch than the no-allocation entry point's fixed buffer holds";
    default: return "unknown status";
    }
}

int palimpsa_version(void) { return PALIMPSA_VERSION; }

}  // extern "C"
