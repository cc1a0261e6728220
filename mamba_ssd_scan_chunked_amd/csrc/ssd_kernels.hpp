// SSD chunked-scan forward kernel for gfx950 (MI355X).
//
// ssd_scan_kernel, one workgroup per (row, head), P/16 waves; wave w owns
// channels p in [16w, 16w+16).  The workgroup walks its row block by block
// (QB = 32 or 64 tokens) with the P x N state held in MFMA accumulator
// registers for the whole row.  Per block:
//   a. log-decay l_t = dt_t A_h (kept in log2 units) and its inclusive
//      cumulative sum within the block, by a wavefront scan
//      (the within-chunk cumsum of the chunked algorithm);
//   b. C B^T over the causal 16x16 tiles of the block on bf16 MFMA, from the
//      C and B tiles staged in LDS, shared out over the waves (the intra-chunk
//      C B^T products of the dual form Y = [L o (C B^T)] X, "088 Mamba-2",
//      section 2.2; the diagonal-block step of key design 2 on the
//      "Mamba-2 - Transformer and SSM share one algebra" page);
//   c. masked decay L[t][s] = exp(cum_t - cum_s) for s <= t in the same
//      sequence, else 0, applied to those tiles in registers (segment sum,
//      section 2.2) and left in LDS as bf16;
//   d. y_diag = (L o CB) X on bf16 MFMA (diagonal block, section 2.3);
//   e. y_off  = exp(cum_t) C_t H_prev, the incoming state read out by C and
//      decayed to each position (left factor, section 3 of "088 Mamba-2");
//   f. H <- exp(cum_end) H + X^T (exp(cum_end - cum_s) o B), the block's end
//      state combined with the carried one (right factor and the
//      inter-chunk scan step real_end = block_decay * prev + local_end);
//   g. y = y_off + y_diag + D x, written once to HBM in fp32.
// Sequence boundaries inside a block (seq_idx) split it into segments:
// L is masked across segments, each segment's incoming state is either the
// carried state or its own initial state, and the state of a sequence that
// ends inside the block is written to final_state on the spot.
//
// Because the state stays in registers, x is read once and y written once;
// the only other traffic is dt and the per-block B and C tiles, which all
// heads of a group read through L2.

#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ssd {

// Cache-policy bits of the buffer loads and stores (gfx950: 1 = sc0, 2 = nt,
// 16 = sc1).  y is written once and never read back by the kernel: its stores are
// non-temporal at device scope (nt | sc1), so its stream does not displace the B
// and C rows that the heads of a row share in L2.  x loads keep the default policy
// (a sweep of nt, sc0 and sc1 on them changed nothing measurable).
constexpr int kXLoadPolicy = 0;
constexpr int kYStorePolicy = 18;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- MFMA traits
// 16x16 output tiles.  Accumulator layout (both types): lane l holds rows
// 4*(l/16) + i, i = 0..3, of column l % 16.  Operand layout: lane l holds row
// (A) or column (B) l % 16 and K values KPL*(l/16) .. KPL*(l/16)+KPL-1 of the
// KSTEP-wide step.
template <typename TI> struct Mfma;
template <> struct Mfma<__bf16> {
    static constexpr int KPL = 8, KSTEP = 32;
    typedef bf16x8 frag;
    __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    static constexpr int KPL = 1, KSTEP = 4;
    typedef float frag;
    __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

template <typename TI> __device__ inline TI to_in(float v);
template <> __device__ inline __bf16 to_in<__bf16>(float v) { return (__bf16)v; }
template <> __device__ inline float to_in<float>(float v) { return v; }
__device__ inline float to_f32(__bf16 v) { return (float)v; }
__device__ inline float to_f32(float v) { return v; }

// K-contiguous fragment from LDS (16-byte aligned for bf16).
template <typename TI> __device__ inline typename Mfma<TI>::frag lds_frag(const TI* p);
template <> __device__ inline bf16x8 lds_frag<__bf16>(const __bf16* p) { return *(const bf16x8*)p; }
template <> __device__ inline float lds_frag<float>(const float* p) { return *p; }

__device__ inline float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// Step size from the dt input: dt + bias, optionally through softplus(v) =
// log(1 + e^v) (the Mamba block's step-size map, simplified block pseudocode
// of the "Mamba" paper story), as max(v, 0) + log1p(t) with t = e^-|v| in
// (0, 1], so that nothing overflows.  log1p(t) comes from the hardware exp2
// and log2 with Goldberg's correction for the rounding of u = 1 + t
// (log1p(t) = log(u) t / (u - 1), and t itself when u rounds to 1; "What every
// computer scientist should know about floating-point arithmetic", 1991,
// theorem 4).  Relative error below 4e-6 down to v = -80 (below 1e-6 for
// |v| <= 12), nearly all from rounding |v| log2(e) before the exp2, in about
// ten instructions against some sixty and two branches for the library's log1p.
__device__ inline float step_size(float v, int softplus) {
    if (!softplus) return v;
    const float t = __builtin_amdgcn_exp2f(-fabsf(v) * 1.4426950408889634f);
    const float u = 1.f + t;
    const float l = u == 1.f ? t : __builtin_amdgcn_logf(u) * 0.6931471805599453f * (t * __builtin_amdgcn_rcpf(u - 1.f));
    return fmaxf(v, 0.f) + l;
}

// Factor on x_t in the state write: 1, the step size (Euler), or the exact
// zero-order hold (exp(Delta A) - 1) / A of h' = A h + B x over one step with
// x and B held (the hold named in section 2 of "Mamba and state space
// models").  A < 0 always (A = -exp(A_log)).
__device__ inline float x_factor(float dtv, float A, int mode) {
    return mode == 2 ? expm1f(dtv * A) / A : (mode == 1 ? dtv : 1.f);
}

// Rows of the state tiles.  The state S (P x N) is held transposed, S^T[n][p],
// as N/16 accumulator tiles per wave; accumulator row rho = 4*(l/16) + i of
// tile m holds state row n = nrow(m, rho).  For N % 32 == 0 the rows of tile
// pairs (2k, 2k+1) are interleaved so that lane group l/16 of the pair holds
// the 8 consecutive rows 32k + 8*(l/16) .. +7: converted to bf16 they are
// exactly the B operand of the read-out C . S^T for the K step k, and the A
// operand (C) is one contiguous 16-byte read.  The permutation is applied to
// the rows of the B^T operand that produces the state, so no data moves.
template <int N>
__device__ inline int nrow(int m, int rho) {
    if constexpr (N % 32 == 0) return 32 * (m >> 1) + 8 * (rho >> 2) + 4 * (m & 1) + (rho & 3);
    else return 16 * m + rho;
}

// K steps of the read-out product C . S^T (K = N).
template <typename TI, int N> struct OffK {
    static constexpr int NK = N / Mfma<TI>::KSTEP;
};

// B-operand fragments of the read-out from MT state accumulator tiles (a whole
// state or the half a wave owns): bf16 tile pair (2k, 2k+1) is fragment k;
// fp32 element i of tile m is fragment 4m + i.
template <int MT>
__device__ inline void state_frags(const f32x4 (&st)[MT], bf16x8 (&sf)[MT / 2]) {
#pragma unroll
    for (int k = 0; k < MT / 2; ++k) {
        bf16x8 f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[i] = (__bf16)st[2 * k][i];
            f[4 + i] = (__bf16)st[2 * k + 1][i];
        }
        sf[k] = f;
    }
}
template <int MT>
__device__ inline void state_frags(const f32x4 (&st)[MT], float (&sf)[4 * MT]) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) sf[4 * m + i] = st[m][i];
}

// Same fragments from an fp32 state row in global memory (row p = this lane's channel).
template <int N>
__device__ inline void global_state_frags(const float* row, int lg, bf16x8 (&sf)[N / 32]) {
#pragma unroll
    for (int k = 0; k < N / 32; ++k) {
        const float4 lo = *(const float4*)(row + 32 * k + 8 * lg);
        const float4 hi = *(const float4*)(row + 32 * k + 8 * lg + 4);
        bf16x8 f;
        f[0] = (__bf16)lo.x; f[1] = (__bf16)lo.y; f[2] = (__bf16)lo.z; f[3] = (__bf16)lo.w;
        f[4] = (__bf16)hi.x; f[5] = (__bf16)hi.y; f[6] = (__bf16)hi.z; f[7] = (__bf16)hi.w;
        sf[k] = f;
    }
}
template <int N>
__device__ inline void global_state_frags(const float* row, int lg, float (&sf)[N / 4]) {
#pragma unroll
    for (int m = 0; m < N / 16; ++m) {
        const float4 v = *(const float4*)(row + nrow<N>(m, 4 * lg));
        sf[4 * m + 0] = v.x; sf[4 * m + 1] = v.y; sf[4 * m + 2] = v.z; sf[4 * m + 3] = v.w;
    }
}

// A-operand fragment of the read-out: row t of the C tile at the K indices of step k.
template <int N>
__device__ inline bf16x8 c_frag(const __bf16* row, int k, int lg) { return *(const bf16x8*)(row + 32 * k + 8 * lg); }
template <int N>
__device__ inline float c_frag(const float* row, int k, int lg) { return row[nrow<N>(k >> 2, 4 * lg + (k & 3))]; }

// XOR swizzle of the bf16 B and X tiles in LDS.  Row r of a tile keeps its
// 8-byte units (four bf16), unit u at position u ^ swz(r) (only the low five
// bits of u change, so a unit stays in its 256-byte span of the row).  swz is
// linear over GF(2): for row indices with disjoint bits, swz(a + b) = swz(a) ^
// swz(b), so the part that is a compile-time constant folds away.  The masks
// were chosen by an exhaustive bank model of the tiles' accesses (the 16-byte
// row writes, the transposing reads of the state update, the row reads of
// C B^T and of the skip term): they leave the B tile free of bank conflicts
// for N = 128 (within 1.25x of it for N = 256) and the X tile within 1.35x for
// 80-channel workgroups, against 2x (B) and 1.8x (X) for the padded layout.
__device__ inline int swz(int r) {
    return (__builtin_popcount(r & 7) & 1) | ((__builtin_popcount(r & 50) & 1) << 1) |
           ((__builtin_popcount(r & 6) & 1) << 2) | ((__builtin_popcount(r & 28) & 1) << 3) |
           ((__builtin_popcount(r & 5) & 1) << 4);
}
// Element offset of unit u of row r in a tile of pitch lp elements.
template <bool SW>
__device__ inline int unit_off(int r, int u, int lp) { return r * lp + 4 * (SW ? (u ^ swz(r)) : u); }

// Operand fragment of X^T (row = channel p0 + l%16, K = tokens ks + KPL*(l/16) ..)
// read from a row-major tile sX[t][p] (pitch lp elements).  bf16: the LDS
// transpose read; within each group of 16 lanes, lane j reads 4 channels
// p0 + 4(j%4) .. of token row R + j/4, and the hardware hands lane i channel
// p0 + i of rows R .. R+3; two reads give the 8 tokens of one K step.
// fp32: one value per lane, no transpose needed.
typedef short i16x4 __attribute__((ext_vector_type(4)));
template <bool SW = false>
__device__ inline bf16x8 x_frag(const __bf16* sX, int lp, int ks, int p0, int lr, int lg) {
    const int rl = 8 * lg + (lr >> 2), u = (p0 >> 2) + (lr & 3);
    const __bf16* a = SW ? sX + unit_off<SW>(ks + rl, u, lp) : sX + (ks + rl) * lp + p0 + 4 * (lr & 3);
    const __bf16* a4 = SW ? sX + unit_off<SW>(ks + 4 + rl, u, lp) : a + 4 * lp;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a4);
    const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
    return __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <bool SW = false>
__device__ inline float x_frag(const float* sX, int lp, int ks, int p0, int lr, int lg) {
    return sX[(ks + lg) * lp + p0 + lr];
}

// The same operand with every token t scaled by wt(t) (and rounded once to the
// input type): the K values a lane holds are tokens ks + KPL*(l/16) + e.
template <bool SW = false, typename F>
__device__ inline bf16x8 weighted_x_frag(const __bf16* sX, int lp, int ks, int p0, int lr, int lg, F wt) {
    const bf16x8 x = x_frag<SW>(sX, lp, ks, p0, lr, lg);
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)(wt(ks + 8 * lg + e) * (float)x[e]);
    return r;
}
template <bool SW = false, typename F>
__device__ inline float weighted_x_frag(const float* sX, int lp, int ks, int p0, int lr, int lg, F wt) {
    return wt(ks + lg) * x_frag(sX, lp, ks, p0, lr, lg);
}
// An operand whose K values are tokens (K = token ks + KPL*(l/16) + e), with the
// tokens for which keep() is false replaced by zero.  A select, not a product
// with zero, so that an Inf or NaN of another sequence stays out of the sum.
template <typename F>
__device__ inline bf16x8 mask_frag(const bf16x8& v, int ks, int lg, F keep) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = keep(ks + 8 * lg + e) ? v[e] : (__bf16)0.f;
    return r;
}
template <typename F>
__device__ inline float mask_frag(float v, int ks, int lg, F keep) { return keep(ks + lg) ? v : 0.f; }
// An X operand already in registers, weighted the same way.
template <typename F>
__device__ inline bf16x8 weight_frag(const bf16x8& x, int ks, int lg, F wt) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)(wt(ks + 8 * lg + e) * (float)x[e]);
    return r;
}

// B tile in LDS: row t holds the N values of token t, pitch LB elements: N + 4
// (8-byte aligned rows), or N with the swizzle above for bf16 and N >= 128.

// A operand of the state update for state tile m and the K step of tokens
// ks .. ks+KSTEP-1: row rho = l % 16 is state row n = nrow(m, rho), K values are
// tokens ks + KPL*(l/16) + 0 .. KPL-1.  bf16: two transposing reads of the
// token-major B tile; lane j of each 16-lane group loads the four values
// n = nrow(m, 4(j%4)) .. +3 of token ks + 8(l/16) + j/4 (+4 for the second read)
// and the hardware hands lane i row nrow(m, i) of those four tokens.
template <int N, int LB, bool SW = false>
__device__ inline bf16x8 bt_frag(const __bf16* sB, int m, int ks, int lr, int lg) {
    const int rl = 8 * lg + (lr >> 2), u = nrow<N>(m, 4 * (lr & 3)) >> 2;
    const __bf16* lo = SW ? sB + unit_off<SW>(ks + rl, u, LB) : sB + (ks + rl) * LB + nrow<N>(m, 4 * (lr & 3));
    const __bf16* l4 = SW ? sB + unit_off<SW>(ks + 4 + rl, u, LB) : lo + 4 * LB;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)lo);
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)l4);
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, b), 0, 1, 2, 3, 4, 5, 6, 7);
}
template <int N, int LB, bool SW = false>
__device__ inline float bt_frag(const float* sB, int m, int ks, int lr, int lg) {
    return sB[(ks + lg) * LB + nrow<N>(m, lr)];
}

// Operand of C B^T holding B row s at the K indices n of step k (natural order):
// bf16 n = 32k + 8(l/16) .. +7 (two 8-byte reads); fp32 n = 4k + l/16.
template <int N, int LB, bool SW = false>
__device__ inline bf16x8 brow_frag(const __bf16* sB, int s, int k, int lg) {
    const int u = 8 * k + 2 * lg;
    const __bf16* r0 = SW ? sB + unit_off<SW>(s, u, LB) : sB + s * LB + 32 * k + 8 * lg;
    const __bf16* r1 = SW ? sB + unit_off<SW>(s, u + 1, LB) : r0 + 4;
    const bf16x4 a = *(const bf16x4*)r0;
    const bf16x4 b = *(const bf16x4*)r1;
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <int N, int LB, bool SW = false>
__device__ inline float brow_frag(const float* sB, int s, int k, int lg) {
    return sB[s * LB + 4 * k + lg];
}
// Operand of C B^T holding C row t at the same K indices (natural order).
template <int N>
__device__ inline bf16x8 crow_frag(const __bf16* row, int k, int lg) { return *(const bf16x8*)(row + 32 * k + 8 * lg); }
template <int N>
__device__ inline float crow_frag(const float* row, int k, int lg) { return row[4 * k + lg]; }

// Make this wave's LDS writes visible to its own other lanes.
__device__ inline void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global
// memory, which makes every wave wait for all of its outstanding global loads
// (the prefetches of the next blocks) at each barrier; the tiles exchanged
// through barriers here all live in LDS.
__device__ inline void block_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Raw buffer resources: loads outside [0, bytes) return zero and stores there
// are dropped by the hardware range check, so the ragged last block needs no
// per-element guards (and no divergent branches around memory operations).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int64_t lim = bytes < 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)lim, 0x00020000);
}
template <int AUX = 0>
__device__ inline uint4 buf_load16(rsrc_t r, int off) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline uint2 buf_load8(rsrc_t r, int off) {
    typedef unsigned int u2 __attribute__((ext_vector_type(2)));
    const u2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_uint2(v.x, v.y);
}
__device__ inline float buf_load_f32(rsrc_t r, int off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline int buf_load_i32(rsrc_t r, int off) {
    return __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
template <int AUX = 0>
__device__ inline void buf_store16(f32x4 v, rsrc_t r, int off) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, off, 0, AUX);
}

// Scheduling hint for a straight-line stretch of LDS-fed MFMAs: keep LEAD LDS
// reads ahead of the MFMA that consumes them, then alternate one MFMA with RPM
// reads.  Without it the scheduler issues each operand read right before its
// MFMA and waits for it, exposing the full LDS latency on every product.
template <int LEAD, int NMFMA, int RPM>
__device__ inline void pipeline_lds_mfma() {
    __builtin_amdgcn_sched_group_barrier(0x100, LEAD, 0);
#pragma unroll
    for (int i = 0; i < NMFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
    }
}

struct ScanParams {
    const void* x;
    const float* dt;
    const float* A_log;
    const float* D;
    const float* init;
    const int32_t* seq_idx;
    float* y;
    float* fin;
    const void* B;
    const void* C;
    int64_t batch, T, H, G, nseqs;
    int nblk;
    const float* dt_bias;   // (H) added to dt before the step-size map, or null
    int dt_softplus;        // step size softplus(dt + dt_bias) instead of dt + dt_bias
    int x_scale;            // factor on x in the state write: 0 none, 1 step size, 2 zero-order hold
    // A row may be split into nseg segments of seg_blocks blocks that run in
    // parallel: a local pass gives each segment but the last its end state from
    // a zero incoming state and the decay it carries across, a combine step
    // turns those into every segment's incoming state, and the scan proper then
    // starts each segment from it.
    int seg_blocks;     // blocks per segment (the whole row when nseg == 1)
    int nseg;           // segments per row
    float* seg_state;   // (batch, H, nseg-1, P, N): local end states, then incoming states of segments 1..
    float* seg_carry;   // (batch, H, nseg-1): decay factor across each segment (0 if a sequence starts in it)
};

struct CombineParams {
    const float* init;
    const int32_t* seq_idx;
    float* seg_state;
    const float* seg_carry;
    int64_t batch, T, H, nseqs;
    int P, N, nseg;
};

// ============================================================== recurrent step
// One token of the recurrence per (row, head), on the fp32 state in place:
// S <- a S + x B^T, y = S C + D x, a = exp(dt A) (the recurrence of "088
// Mamba-2", section 2.1, one step; the decay of the selective-SSM section of
// the Mamba story; the skip term of section 2 of "Mamba and state space
// models").  Bound by the state's HBM read and write.
struct StepParams {
    const void* x;          // (batch, H, P)
    const float* dt;        // (batch, H)
    const float* A_log;     // (H)
    const void* B;          // (batch, G, N)
    const void* C;          // (batch, G, N)
    const float* D;         // (H) or null
    float* state;           // (batch, H, P, N), updated in place
    float* y;               // (batch, H, P)
    int64_t batch, H, G;
    const float* dt_bias;   // (H) or null
    int dt_softplus;        // as in ScanParams
    int x_scale;            // as in ScanParams
};

// One workgroup of 256 threads per (row, head).  The head's state is P rows of
// L = N/4 float4s; in pass j thread t handles float4 f = 256 j + t, i.e. row
// p = f / L and columns n = 4c .. 4c+3 with c = t % L, the same columns in every
// pass, so B and C are read once per thread.  Each pass reads and writes 4 KB
// of contiguous state per workgroup (64 lanes x 16 bytes per instruction), and
// the read-out of row p is summed over its L lanes (consecutive in the wave) by
// a fixed butterfly, so y is deterministic.
template <typename TI, int P, int N>
__global__ __launch_bounds__(256) void ssd_step_kernel(StepParams prm) {
    constexpr int L = N / 4, F = P * N / 4, J = (F + 255) / 256;
    static_assert(N % 4 == 0 && L <= 64 && 64 % L == 0 && F >= 64, "step shape");
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / prm.H, h = bh % prm.H;
    const int64_t g = h / (prm.H / prm.G);
    const int tid = threadIdx.x, c = tid % L;
    const float A = -expf(prm.A_log[h]);
    const float dtv = step_size(prm.dt[bh] + (prm.dt_bias ? prm.dt_bias[h] : 0.f), prm.dt_softplus);
    const float a = expf(dtv * A);
    const float xf = x_factor(dtv, A, prm.x_scale);              // input scaling (D uses the unscaled x)
    const float Dh = prm.D ? prm.D[h] : 0.f;
    const TI* Bg = (const TI*)prm.B + (b * prm.G + g) * N + 4 * c;
    const TI* Cg = (const TI*)prm.C + (b * prm.G + g) * N + 4 * c;
    float bv[4], cv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bv[e] = to_f32(Bg[e]);
        cv[e] = to_f32(Cg[e]);
    }
    float4* st = (float4*)(prm.state + bh * P * N);
    const TI* xr = (const TI*)prm.x + bh * P;
    float4 sv[J];
    float xv[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {                                // every load issued before any store
        const int f = 256 * j + tid;
        if (F % 256 == 0 || f < F) {
            sv[j] = st[f];
            xv[j] = to_f32(xr[f / L]);
        }
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int f = 256 * j + tid;
        if (F % 256 == 0 || f < F) {                             // whole rows, so whole butterfly groups
            const float xs = xf * xv[j];
            float4 v = sv[j];
            v.x = a * v.x + xs * bv[0];
            v.y = a * v.y + xs * bv[1];
            v.z = a * v.z + xs * bv[2];
            v.w = a * v.w + xs * bv[3];
            st[f] = v;
            float acc = cv[0] * v.x + cv[1] * v.y + cv[2] * v.z + cv[3] * v.w;
#pragma unroll
            for (int d = L / 2; d >= 1; d >>= 1) acc += __shfl_xor(acc, d);
            if (c == 0) prm.y[bh * P + f / L] = acc + Dh * xv[j];
        }
    }
}

// ============================================================== scan kernel
template <typename TI> struct CumType { typedef float type; };
template <> struct CumType<float> { typedef double type; };   // fp32 path: exponent differences in fp64

// Inclusive prefix sum over the 64 lanes of a wavefront: Hillis-Steele steps
// inside each row of 16 lanes (DPP row shifts), then the row totals are
// broadcast into the following rows.
template <int CTRL, int RMASK>
__device__ inline float dpp_add(float x) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, RMASK, 0xf, true);
    return x + __builtin_bit_cast(float, t);
}
__device__ inline float wave_incl_scan(float x) {
    x = dpp_add<0x111, 0xf>(x);   // row_shr:1
    x = dpp_add<0x112, 0xf>(x);   // row_shr:2
    x = dpp_add<0x114, 0xf>(x);   // row_shr:4
    x = dpp_add<0x118, 0xf>(x);   // row_shr:8
    x = dpp_add<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
    x = dpp_add<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}
__device__ inline double wave_incl_scan(double x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const double o = __shfl_up(x, d);
        if (lane >= d) x += o;
    }
    return x;
}

// SPW: 16-channel slices per workgroup.  By default a workgroup holds one head
// (SPW = P / 16); with more, it holds SPW consecutive slices of a row, which
// may belong to two heads (consecutive slices are consecutive channels of the
// flattened (head, channel) dimension).
template <typename TI, int P, int N, int QB, int SPW_ = P / 16>
struct ScanCfg {
    static constexpr int SZ = (int)sizeof(TI);
    static constexpr int VE = 16 / SZ;                // elements per 16-byte vector
    static constexpr int KPL = Mfma<TI>::KPL, KSTEP = Mfma<TI>::KSTEP;
    static constexpr int NK = OffK<TI, N>::NK;        // K steps of the read-out over the state dimension
    static constexpr int RT = QB / 16;                // token tiles of a block
    static constexpr int MT = N / 16;                 // state tiles of one 16-channel slice
    static constexpr int NPT = P / 16;                // 16-channel slices of a head
    static constexpr int SPW = SPW_;                  // slices of this workgroup
    static constexpr int MLH = SPW % NPT == 0 ? SPW / NPT : (SPW + NPT - 2) / NPT + 1;   // heads it may touch
    static constexpr int XW = 16 * SPW;               // channels of the workgroup's X tile
    // Each slice is shared by NH waves: wave (slice pt, half nh) owns state tiles
    // [nh MT/NH, (nh+1) MT/NH) (whole K steps of the read-out) and token tiles
    // own_tile(nh, i) of the outputs.
    static constexpr int NH = (SZ == 2 ? MT % 4 == 0 : MT % 2 == 0) && RT % 2 == 0 ? 2 : 1;
    static constexpr int NW = SPW * NH;
    static constexpr int NT = NW * 64;
                                                      // (the sequence-id variants, whose segment path
                                                      // needs more registers, are left at two)
    static constexpr int MTH = MT / NH, NKH = NK / NH, RTH = RT / NH;
    static constexpr int LC = N + VE;                 // pitch of C rows (elements)
    // Swizzled B and X tiles (bf16).  Their addresses cost registers, so they are
    // used only for five-slice workgroups with N = 128 and 64-token blocks (one
    // workgroup per CU, three waves per SIMD: 168 VGPRs); elsewhere they spill.
    static constexpr bool SWB = SZ == 2 && N == 128 && SPW_ == 5 && QB == 64;
    static constexpr bool SWX = SWB;
    static constexpr int LB = SWB ? N : N + 4;        // pitch of B rows
    static constexpr int LQ = QB + VE;                // pitch of the rows of L o CB (indexed by token s)
    static constexpr int LR = SWX ? 128 : XW + 32 / SZ;  // pitch of the row-major X tile (fp32: 32 bytes of pad:
                                                      // the four rows of a transposed read fall in
                                                      // distinct banks)
    static_assert(!SWX || XW <= 128, "a swizzled X row holds at most 128 channels");
    static constexpr int NTILE = RT * (RT + 1) / 2;   // causal 16x16 tiles of L o CB
    static constexpr int TPW = (NTILE + NW - 1) / NW; // causal tiles per wave (surplus slots repeat a tile)
    // LDS tiles: C, B (both token-major), masked decay L o CB, X (row-major; the
    // state update weights it per token in registers) and, with NH = 2, each wave's
    // half of the state as read-out operands
    static constexpr int OFF_C = 0;
    static constexpr int OFF_B = OFF_C + QB * LC;
    static constexpr int OFF_LM = OFF_B + QB * LB;
    static constexpr int OFF_XR = OFF_LM + MLH * QB * LQ;            // L o CB of each head
    static constexpr int OFF_SX = OFF_XR + QB * LR;
    static constexpr int BUF_ELEMS = OFF_SX + (NH > 1 ? NW * NKH * 64 * KPL : 0);
    // workgroups per CU that the LDS footprint allows (the tiles plus about 1 KB per
    // head and 1.5 KB of other per-token arrays), at most 2; and the waves per SIMD
    // to plan registers for: one head per workgroup, two workgroups per CU, else
    // that many workgroups
    static constexpr int WGPC = 163840 / (BUF_ELEMS * SZ + MLH * 1024 + 1536) >= 2 ? 2 : 1;
    static constexpr int WPE = SPW == NPT ? (NW >= 8 ? NW / 2 : 2) : (WGPC * NW + 3) / 4;
    // per-thread work units
    static constexpr int CV = QB * N / VE, CPT = (CV + NT - 1) / NT;           // C (and B) tile vectors
    static constexpr int XU = QB * XW / VE, XPT = (XU + NT - 1) / NT;           // 16-byte pieces of the X tile
    // token tile i of the outputs of half nh: the causal work of the diagonal
    // block is split evenly ({0, 3} and {1, 2} of four tiles)
    __device__ static inline int own_tile(int nh, int i) {
        if constexpr (NH == 1) return i;
        else if constexpr (RT == 2) return nh;
        else return i == 0 ? nh : 3 - nh;
    }
};

// LOCAL: the local pass over segments 0 .. nseg-2 (end state from a zero incoming
// state and the carried decay, no outputs); otherwise the scan proper.
template <typename TI, int P, int N, int QB, bool SEQ, bool XSCALE, bool LOCAL, int SPW = P / 16>
__global__ __attribute__((amdgpu_flat_work_group_size(1, ScanCfg<TI, P, N, QB, SPW>::NT),
                          amdgpu_waves_per_eu(SEQ && SPW == P / 16 ? 2 : ScanCfg<TI, P, N, QB, SPW>::WPE)))
void ssd_scan_kernel(ScanParams prm) {
    typedef ScanCfg<TI, P, N, QB, SPW> K;
    typedef Mfma<TI> MF;
    typedef typename MF::frag frag;
    typedef typename CumType<TI>::type cum_t;
    constexpr int NT = K::NT, VE = K::VE, LC = K::LC, LB = K::LB, LQ = K::LQ, LR = K::LR, KPL = K::KPL;
    constexpr int KSTEP = K::KSTEP, SZ = K::SZ, NK = K::NK, RT = K::RT, MT = K::MT, NW = K::NW;
    constexpr int NH = K::NH, NPT = K::NPT, MTH = K::MTH, NKH = K::NKH, RTH = K::RTH, MLH = K::MLH, XW = K::XW;
    constexpr int NFH = SZ == 2 ? MTH / 2 : 4 * MTH;               // read-out fragments of a state half
    constexpr bool LEADER_SCAN = true;     // without sequence ids only the head leaders run the per-token scan
    static_assert(NFH == NKH, "fragments of a state half are whole K steps");
    static_assert(QB <= 64 && QB % KSTEP == 0 && QB % 16 == 0, "block length");
    static_assert(N % KSTEP == 0 && N % 16 == 0 && P % 16 == 0, "shape");

    __shared__ __attribute__((aligned(16))) TI smem[K::BUF_ELEMS];
    // per-token scalars of the block, shared by all waves (written by wave 0)
    constexpr int SQ = SEQ ? 1 : 0, EU = XSCALE ? 1 : 0;
    // (one copy per head of the workgroup, written by that head's first wave)
    __shared__ __attribute__((aligned(16))) cum_t sCumH[MLH][64];      // cumulative log2 decay
    __shared__ __attribute__((aligned(16))) float sRowH[MLH][64];      // read-out row scale
    __shared__ __attribute__((aligned(16))) float sWxH[MLH][64];       // end-state weight exp2(cum_end - cum) (dt)
    __shared__ __attribute__((aligned(16))) float sDtfH[MLH][64 * EU + 4];   // factor on x_t (input scaling)
    __shared__ __attribute__((aligned(16))) int sSeg[64 * SQ + 4];     // segment of each token
    __shared__ int sStart[65 * SQ + 1];
    __shared__ int sSeqOf[65 * SQ + 1];

    TI* sC = smem + K::OFF_C;
    TI* sB = smem + K::OFF_B;
    TI* sXr = smem + K::OFF_XR;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: wave-level values stay scalar
    const int lr = lane & 15, lg = lane >> 4;
    const int ls = w % SPW, nh = w / SPW;     // this wave's slice of the workgroup, and its half of the state
    const int xc = 16 * ls;                   // its channels in the X tile
    const int mb = nh * MTH;                  // first state tile this wave owns
    const int kbo = nh * NKH, kbp = (1 - nh) * NKH;   // read-out K steps of its half and of the partner's
    // this wave's and its partner's read-out fragments in the exchange area (16-byte slots per lane)
    TI* sxo = smem + K::OFF_SX + ((ls * NH + nh) * NKH * 64 + lane) * KPL;
    const TI* sxp = smem + K::OFF_SX + ((ls * NH + (NH - 1 - nh)) * NKH * 64 + lane) * KPL;

    // Work-item order: runs of consecutive (row, slice group) items go to the same
    // XCD (workgroups are dealt round-robin over the 8 XCDs), so the heads of
    // a row share that row's B and C tiles in one L2.
    const int64_t T = prm.T, H = prm.H, G = prm.G;
    const int64_t nsg = H * NPT / SPW;                           // slice groups per row
    const int nsl = LOCAL ? prm.nseg - 1 : prm.nseg;             // segments this launch covers
    const int64_t units = prm.batch * nsg * nsl;
    int64_t u = blockIdx.x;
    if (units % 8 == 0) u = (int64_t)(blockIdx.x % 8) * (units / 8) + blockIdx.x / 8;
    const int64_t grp = u % nsg, rowseg = u / nsg;
    const int sg = (int)(rowseg % nsl);
    const int64_t b = rowseg / nsl;
    const int64_t gs0 = grp * SPW;                               // first slice of the workgroup in its row
    const int64_t h = (gs0 + ls) / NPT;                          // this wave's head and channels
    const int pt = (int)((gs0 + ls) % NPT), p0 = 16 * pt;
    const int64_t hf = gs0 / NPT;                                // first head of the workgroup
    const int lh = (int)(h - hf), nlh = (int)((gs0 + SPW - 1) / NPT - hf) + 1;
    const bool head_leader = nh == 0 && (ls == 0 || pt == 0);   // publishes its head's per-token scalars
    const int64_t g = hf / (H / G);
    cum_t* sCum = sCumH[lh];
    float* sRow = sRowH[lh];
    float* sWx = sWxH[lh];
    float* sDtf = sDtfH[lh];
    TI* sLmH = smem + K::OFF_LM;                                 // L o CB of local head l at l * QB * LQ
    TI* sLm = sLmH + lh * QB * LQ;
    const int blk0 = sg * prm.seg_blocks;
    const int blk1 = min(prm.nblk, blk0 + prm.seg_blocks);
    const int64_t slot = (b * H + h) * (prm.nseg - 1) + sg;     // this segment's local-pass slot

    // A_h in log2 units, so that every decay is exp2 of a cumulative sum
    cum_t A2;
    if constexpr (sizeof(cum_t) == 8) A2 = -exp((double)prm.A_log[h]) * 1.4426950408889634;
    else A2 = -expf(prm.A_log[h]) * 1.4426950408889634f;
    const float Dh = prm.D ? prm.D[h] : 0.f;
    const float dtb = prm.dt_bias ? prm.dt_bias[h] : 0.f;
    const float Anat = -expf(prm.A_log[h]);                      // A_h for the zero-order-hold factor
    const int32_t* seqg = SEQ ? prm.seq_idx + b * T : nullptr;
    auto clamp_seq = [&](int s) { return s < 0 ? 0 : (s >= prm.nseqs ? (int)prm.nseqs - 1 : s); };

    // byte strides between consecutive tokens (the host keeps QB of them below 2^31)
    const int xs = (int)(H * P * SZ), ys = (int)(H * P * 4), cs = (int)(G * N * SZ), ds = (int)(H * 4);
    // row bases; block blk starts QB tokens further, and everything past the
    // row's last token reads as zero / is not written (buffer range check)
    const char* xrow = (const char*)prm.x + ((b * T) * H * P + gs0 * 16) * SZ;
    const char* yrow = (const char*)prm.y + ((b * T) * H * P + gs0 * 16) * 4;
    const char* crow = (const char*)prm.C + ((b * T) * G + g) * N * SZ;
    const char* brow = (const char*)prm.B + ((b * T) * G + g) * N * SZ;
    const char* drow = (const char*)prm.dt + ((b * T) * H + h) * 4;
    const int64_t xrec = ((T - 1) * H * P + XW) * SZ, yrec = ((T - 1) * H * P + XW) * 4;
    const int64_t crec = ((T - 1) * G + 1) * N * SZ, drec = ((T - 1) * H + 1) * 4;

    // ---- initial state of the row's first sequence: this wave's tiles of S^T,
    //      rows nrow(mb + j, 4*lg+i) of channel p0 + lr
    // (a later segment continues the sequence of the token before it; its incoming
    // state is the combined one, and the local pass starts from zero)
    int prevseq = (int)b;
    if (SEQ && T > 0) prevseq = clamp_seq(seqg[blk0 > 0 ? (int64_t)blk0 * QB - 1 : 0]);
    f32x4 st[MTH];
    const float* src0 = nullptr;
    if constexpr (!LOCAL) {
        if (sg > 0) src0 = prm.seg_state + ((slot - 1) * P + p0 + lr) * N;
        else if (prm.init) src0 = prm.init + (((int64_t)prevseq * H + h) * P + p0 + lr) * N;
    }
    if (src0) {
        const float* src = src0;
#pragma unroll
        for (int j = 0; j < MTH; ++j) {
            const float4 v = *(const float4*)(src + nrow<N>(mb + j, 4 * lg));
            st[j] = f32x4{v.x, v.y, v.z, v.w};
        }
    } else {
#pragma unroll
        for (int j = 0; j < MTH; ++j) st[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    auto write_state = [&](const f32x4 (&s)[MTH], int seq) {
        if (!prm.fin) return;
        float* dst = prm.fin + (((int64_t)seq * H + h) * P + p0 + lr) * N;
#pragma unroll
        for (int j = 0; j < MTH; ++j)
            *(float4*)(dst + nrow<N>(mb + j, 4 * lg)) = make_float4(s[j][0], s[j][1], s[j][2], s[j][3]);
    };
    // this wave's half of the state, as read-out operands, for its partner; the
    // same operands are kept for this wave's own next read-out (the state does
    // not change in between)
    frag sfk[NKH];
    auto sx_store = [&]() {
        if constexpr (NH > 1) {
            state_frags<MTH>(st, sfk);
#pragma unroll
            for (int j = 0; j < NKH; ++j) *(frag*)(sxo + j * 64 * KPL) = sfk[j];
        }
    };

    // The upper 16x16 tile next to an even diagonal tile is read by a 32-wide
    // K step of the diagonal product; it is zero and never rewritten.
    if constexpr (KSTEP > 16) {
        for (int v = tid; v < MLH * (RT / 2) * 16 * 16; v += NT) {
            const int l = v / ((RT / 2) * 256), vv = v % ((RT / 2) * 256);
            const int r = 2 * (vv / 256), i = (vv / 16) % 16, c = vv % 16;
            sLmH[l * QB * LQ + (16 * r + i) * LQ + 16 * (r + 1) + c] = to_in<TI>(0.f);
        }
    }
    // Causal tiles (row tile I, column tile J <= I) of L o CB computed by this
    // wave: q = w, w + NW, ... (mod NTILE), q = I (I + 1) / 2 + J.
    int tI[K::TPW], tJ[K::TPW];
#pragma unroll
    for (int j = 0; j < K::TPW; ++j) {
        const int q = (w + j * NW) % K::NTILE;
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= q) ++I;
        tI[j] = I;
        tJ[j] = q - I * (I + 1) / 2;
    }

    // ---- one block of loads, issued at the top of an iteration and consumed
    // at its bottom (after the MFMA phases of the previous block), so no load
    // result lives across the loop back-edge and the wait counts stay exact.
    uint4 cr[K::CPT], br[K::CPT];
    uint4 xr[K::XPT];
    float dtv = 0.f;
    int sqv = 0;
    // (two groups: the B and C tiles, then dt and X, so that the waves do not all
    // queue every load of the block at the same moment)
    auto issue_x = [&](int blk) {
        const int64_t t0 = (int64_t)blk * QB;
        const rsrc_t rx = make_rsrc(xrow + t0 * xs, xrec - t0 * xs);
        const rsrc_t rd = make_rsrc(drow + t0 * ds, drec - t0 * ds);
        if (SEQ || !LEADER_SCAN || head_leader) dtv = buf_load_f32(rd, lane * ds);
        if constexpr (SEQ) sqv = buf_load_i32(make_rsrc(seqg + t0, (T - t0) * 4), lane * 4);
#pragma unroll
        for (int j = 0; j < K::XPT; ++j) {
            const int v = tid + j * NT;
            if (K::XU % NT == 0 || v < K::XU) xr[j] = buf_load16<kXLoadPolicy>(rx, (v / (XW / VE)) * xs + (v % (XW / VE)) * 16);
        }
    };
    auto issue_bc = [&](int blk) {
        const int64_t t0 = (int64_t)blk * QB;
        const rsrc_t rc = make_rsrc(crow + t0 * cs, crec - t0 * cs);
        const rsrc_t rb = make_rsrc(brow + t0 * cs, crec - t0 * cs);
#pragma unroll
        for (int j = 0; j < K::CPT; ++j) {
            const int v = tid + j * NT;
            if (K::CV % NT == 0 || v < K::CV) {
                const int off = (v / (N / VE)) * cs + (v % (N / VE)) * 16;
                if constexpr (!LOCAL) cr[j] = buf_load16(rc, off);
                br[j] = buf_load16(rb, off);
            }
        }
    };

    // per-block values handed from the preparation of a block to its MFMA phases
    int nstart_c = 0, lastseq_c = prevseq;
    float cend_f = 0.f;
    cum_t seg_total = 0;          // log2 decay across the blocks staged so far
    bool seg_reset = false;       // a sequence started in them

    // ---- preparation of a block from the issued loads: tiles into LDS, the
    //      within-block cumulative decay, segments, X and weighted X.  Every wave
    //      computes the per-token scalars in registers (lane = token); wave 0
    //      publishes them for the MFMA phases.
    auto prep_x = [&]() {
        // X (row-major; each thread holds VE channels of one token)
#pragma unroll
        for (int j = 0; j < K::XPT; ++j) {
            const int v = tid + j * NT;
            if (K::XU % NT == 0 || v < K::XU) {
                const int t = v / (XW / VE), c = v % (XW / VE);
                if constexpr (K::SWX) {
                    *(uint2*)(sXr + unit_off<true>(t, 2 * c, LR)) = make_uint2(xr[j].x, xr[j].y);
                    *(uint2*)(sXr + unit_off<true>(t, 2 * c + 1, LR)) = make_uint2(xr[j].z, xr[j].w);
                } else {
                    *(uint4*)(sXr + t * LR + c * VE) = xr[j];
                }
            }
        }
    };
    auto prep = [&](int blk) {
        const int rows = (int)min((int64_t)QB, T - (int64_t)blk * QB);
#pragma unroll
        for (int j = 0; j < K::CPT; ++j) {
            const int v = tid + j * NT;
            if (K::CV % NT == 0 || v < K::CV) {
                const int t = v / (N / VE), c = v % (N / VE);
                if constexpr (!LOCAL) *(uint4*)(sC + t * LC + c * VE) = cr[j];
                if constexpr (K::SWB) {                        // swizzled 8-byte units
                    *(uint2*)(sB + unit_off<true>(t, 2 * c, LB)) = make_uint2(br[j].x, br[j].y);
                    *(uint2*)(sB + unit_off<true>(t, 2 * c + 1, LB)) = make_uint2(br[j].z, br[j].w);
                } else if constexpr (SZ == 2) {
                    TI* d = sB + t * LB + c * VE;          // 8-byte aligned rows
                    *(uint2*)d = make_uint2(br[j].x, br[j].y);
                    *(uint2*)(d + 4) = make_uint2(br[j].z, br[j].w);
                } else {
                    *(uint4*)(sB + t * LB + c * VE) = br[j];
                }
            }
        }
        // Without sequence ids only the head leaders need the per-token values (they
        // publish them; the other waves read the block's decay from LDS)
        if (!SEQ && LEADER_SCAN && !head_leader) return prep_x();
        if (prm.dt_bias || prm.dt_softplus)                        // step size; 0 past the row's end
            dtv = lane < rows ? step_size(dtv + dtb, prm.dt_softplus) : 0.f;
        const cum_t lv = (cum_t)dtv * A2;
        cum_t cum = wave_incl_scan(lv);                            // dt = 0 past the row's end
        int nstart = 0;
        cum_t before = 0;
        if constexpr (SEQ) {
            const int raw = clamp_seq(sqv);
            const int lastv = __shfl(raw, rows - 1);
            const int sq = lane < rows ? raw : lastv;            // padding tokens continue the last sequence
            const int up = __shfl_up(sq, 1);
            const int prev = (lane == 0) ? prevseq : up;
            const bool start = lane < rows && sq != prev;
            const uint64_t mask = __ballot(start);
            nstart = __popcll(mask);
            lastseq_c = __shfl(sq, QB - 1);
            const uint64_t upto = (lane == 63) ? ~0ull : ((2ull << lane) - 1ull);
            const uint64_t mine = mask & upto;
            const int segl = __popcll(mine);
            if (nstart > 0) {
                // a block with sequence starts: each segment's cumulative decay from
                // its own first token, by a scan per segment, so that no step size
                // (an Inf or NaN one included) crosses a sequence start
                cum_t cs = 0;
                for (int j = 0; j <= nstart; ++j) {
                    const cum_t cj = wave_incl_scan(segl == j ? lv : (cum_t)0);
                    cs = segl == j ? cj : cs;
                }
                cum = cs;
            }
            if (w == 0) {
                if (lane < QB) sSeg[lane] = segl;                // all zero for a single-segment block
                if (start) {
                    sStart[segl] = lane;
                    sSeqOf[segl] = sq;
                }
                if (lane == 0) {
                    sStart[0] = 0;
                    sSeqOf[0] = prevseq;
                }
            }
        }
        const cum_t cend = __shfl(cum, QB - 1);
        nstart_c = nstart;
        cend_f = (float)cend;
        seg_total += cend;
        seg_reset |= nstart > 0;
        const float dtf = XSCALE ? x_factor(dtv, Anat, prm.x_scale) : 1.f;
        if (head_leader && lane < QB) {
            sCum[lane] = cum;
            sRow[lane] = fast_exp2((float)(cum - before));
            sWx[lane] = fast_exp2((float)(cend - cum)) * dtf;  // end-state weight of token lane
            if constexpr (XSCALE) sDtf[lane] = dtf;
        }

        prep_x();
    };

    // ---- this wave's causal tiles of L o CB: C B^T on MFMA (as (C B^T)^T, rows s,
    //      columns t, so that each lane holds 4 consecutive s of one token t), then
    //      the masked decay exp2(cum_t - cum_s) for s <= t (else 0) in registers
    //      (times the input factor of token s when x is scaled; zero across sequence segments).
    //      Surplus slots recompute a tile another wave owns and write the same values.
    //      The values are held in registers and written after the state update, so
    //      that no LDS write separates the operand reads of the MFMA phase (the
    //      compiler cannot move a read above a write to the same array).
    typedef typename std::conditional<SZ == 2, bf16x4, f32x4>::type lm_t;
    lm_t lmv[K::TPW][MLH];
    auto lm_phase = [&]() {
        // K step outer, tile inner: consecutive MFMAs go to independent accumulators
        f32x4 cbt[K::TPW];
#pragma unroll
        for (int j = 0; j < K::TPW; ++j) cbt[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < NK; ++k)
#pragma unroll
            for (int j = 0; j < K::TPW; ++j)
                cbt[j] = MF::mma(brow_frag<N, LB, K::SWB>(sB, 16 * tJ[j] + lr, k, lg),
                                 crow_frag<N>(sC + (16 * tI[j] + lr) * LC, k, lg), cbt[j]);
        // the same C B^T tile under the decay of each head of the workgroup
#pragma unroll
        for (int j = 0; j < K::TPW; ++j) {
            const int I = tI[j], J = tJ[j];                      // uniform over the wave
            const int t = 16 * I + lr, s0 = 16 * J + 4 * lg;
            const f32x4 acc = cbt[j];
#pragma unroll
            for (int l = 0; l < MLH; ++l) {
                if (MLH > 1 && l >= nlh) break;
                const cum_t ct = sCumH[l][t];
                cum_t csv[4];
                if constexpr (sizeof(cum_t) == 4) {
                    const float4 c4 = *(const float4*)(&sCumH[l][s0]);
                    csv[0] = c4.x; csv[1] = c4.y; csv[2] = c4.z; csv[3] = c4.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) csv[e] = sCumH[l][s0 + e];
                }
                float val[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lv = fast_exp2((float)(ct - csv[e])) * acc[e];
                    val[e] = (s0 + e <= t) ? lv : 0.f;
                }
                if constexpr (XSCALE) {
                    const float4 d4 = *(const float4*)(&sDtfH[l][s0]);
                    val[0] *= d4.x; val[1] *= d4.y; val[2] *= d4.z; val[3] *= d4.w;
                }
                if constexpr (SEQ) {
                    const int segt = sSeg[t];
                    const int4 sgv = *(const int4*)(&sSeg[s0]);
                    if (sgv.x != segt) val[0] = 0.f;
                    if (sgv.y != segt) val[1] = 0.f;
                    if (sgv.z != segt) val[2] = 0.f;
                    if (sgv.w != segt) val[3] = 0.f;
                }
                if constexpr (SZ == 2) lmv[j][l] = bf16x4{(__bf16)val[0], (__bf16)val[1], (__bf16)val[2], (__bf16)val[3]};
                else lmv[j][l] = f32x4{val[0], val[1], val[2], val[3]};
            }
        }
    };
    auto lm_store = [&]() {
#pragma unroll
        for (int j = 0; j < K::TPW; ++j)
#pragma unroll
            for (int l = 0; l < MLH; ++l) {
                if (MLH > 1 && l >= nlh) break;
                *(lm_t*)(sLmH + l * QB * LQ + (16 * tI[j] + lr) * LQ + 16 * tJ[j] + 4 * lg) = lmv[j][l];
            }
    };

    // ---- MFMA phases, outputs transposed: y^T tiles (rows p0..p0+15, columns t) of
    //      this wave's token tiles; acc holds the scaled read-out of the carried state,
    //      then the diagonal block
    f32x4 acc[RTH];
    constexpr int KS = QB / KSTEP;           // K steps over the tokens of a block

    // X operands of the diagonal product, read before the barrier that ends the MFMA
    // phase and kept across it (bf16 with paired halves); without sequence ids the
    // state update reads them first and weights a copy, so each is read once
    constexpr int DKS = (KSTEP == 32 && NH == 2) ? 2 : 0;
    constexpr bool XD_SHARED = DKS > 0 && !SEQ && QB / KSTEP == DKS;
    frag xd[DKS > 0 ? DKS : 1];

    // read-out of the carried state over all N (this wave's half from its registers,
    // the partner's from the exchange area) and the update of this wave's half
    auto state_phase = [&]() {
        const int nstart = nstart_c;
        frag sfo[NKH], sfp[NKH];
        if constexpr (!LOCAL) {
            if constexpr (NH > 1) {
#pragma unroll
                for (int j = 0; j < NKH; ++j) sfo[j] = sfk[j];
            } else {
                state_frags<MTH>(st, sfo);
            }
        }
        if constexpr (NH > 1 && !LOCAL) {
#pragma unroll
            for (int j = 0; j < NKH; ++j) sfp[j] = *(const frag*)(sxp + j * 64 * KPL);
        }
#pragma unroll
        for (int i = 0; i < RTH; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!SEQ || nstart == 0) {
            // carried state read out by C:  S C^T (K step outer: the token tiles'
            // accumulators alternate, so consecutive MFMAs are independent)
            if constexpr (!LOCAL) {
                const TI* crw[RTH];
#pragma unroll
                for (int i = 0; i < RTH; ++i) crw[i] = sC + (16 * K::own_tile(nh, i) + lr) * LC;
#pragma unroll
                for (int j = 0; j < NKH; ++j)
#pragma unroll
                    for (int i = 0; i < RTH; ++i) acc[i] = MF::mma(sfo[j], c_frag<N>(crw[i], kbo + j, lg), acc[i]);
                if constexpr (NH > 1) {
#pragma unroll
                    for (int j = 0; j < NKH; ++j)
#pragma unroll
                        for (int i = 0; i < RTH; ++i) acc[i] = MF::mma(sfp[j], c_frag<N>(crw[i], kbp + j, lg), acc[i]);
                }
            }
            // state <- exp(cum_end) state + B^T (weighted X)
            const float alpha = fast_exp2(!SEQ && LEADER_SCAN ? (float)sCum[QB - 1] : cend_f);
#pragma unroll
            for (int j = 0; j < MTH; ++j) st[j] *= alpha;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                frag xw;
                if constexpr (XD_SHARED) {
                    xd[ks] = x_frag<K::SWX>(sXr, LR, ks * KSTEP, xc, lr, lg);
                    xw = weight_frag(xd[ks], ks * KSTEP, lg, [&](int t) { return sWx[t]; });
                } else {
                    xw = weighted_x_frag<K::SWX>(sXr, LR, ks * KSTEP, xc, lr, lg, [&](int t) { return sWx[t]; });
                }
#pragma unroll
                for (int j = 0; j < MTH; ++j) st[j] = MF::mma(bt_frag<N, LB, K::SWB>(sB, mb + j, ks * KSTEP, lr, lg), xw, st[j]);
            }
#pragma unroll
            for (int i = 0; i < (LOCAL ? 0 : RTH); ++i) acc[i] *= sRow[16 * K::own_tile(nh, i) + lr];
            // (not for the swizzled five-slice instance, which the hint makes slower)
            if constexpr (!SEQ && !LOCAL && SZ == 2 && !K::SWB) pipeline_lds_mfma<6, K::TPW * NK + RTH * NK + MTH * KS, 2>();
        } else if constexpr (SEQ) {
            // ---- block with sequence starts, one segment at a time
            // (1) read-out of each segment's incoming state
            for (int j = 0; j <= (LOCAL ? -1 : nstart); ++j) {
                const int a = sStart[j];
                const int e = (j < nstart) ? sStart[j + 1] - 1 : QB - 1;
                if (e < a) continue;                         // empty first segment
                if (j > 0 && !prm.init) continue;            // a zero initial state reads out nothing
                frag f[NK];
                if (j > 0) global_state_frags<N>(prm.init + (((int64_t)sSeqOf[j] * H + h) * P + p0 + lr) * N, lg, f);
#pragma unroll
                for (int i = 0; i < RTH; ++i) {
                    const int t = 16 * K::own_tile(nh, i) + lr;
                    const TI* crw = sC + t * LC;
                    f32x4 tmp = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (j == 0) {
#pragma unroll
                        for (int q = 0; q < NKH; ++q) tmp = MF::mma(sfo[q], c_frag<N>(crw, kbo + q, lg), tmp);
                        if constexpr (NH > 1) {
#pragma unroll
                            for (int q = 0; q < NKH; ++q) tmp = MF::mma(sfp[q], c_frag<N>(crw, kbp + q, lg), tmp);
                        }
                    } else {
#pragma unroll
                        for (int k = 0; k < NK; ++k) tmp = MF::mma(f[k], c_frag<N>(crw, k, lg), tmp);
                    }
                    const bool in = sSeg[t] == j;
                    const float sc = sRow[t];
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[i][q] += in ? sc * tmp[q] : 0.f;
                }
            }
            // (2) state at the end of each segment: a sequence that ends inside
            //     the block hands its state to final_state; the last segment's
            //     state is carried on
            if (!LOCAL && sStart[1] == 0) write_state(st, sSeqOf[0]);   // previous sequence ended with the previous block
            for (int j = 0; j <= nstart; ++j) {
                const int a = sStart[j];
                const int e = (j < nstart) ? sStart[j + 1] - 1 : QB - 1;
                if (e < a) continue;
                // end-of-segment weights: exp2(cum_e - cum_t) (dt) for the segment's tokens, else 0
                const cum_t ce = sCum[e];
                auto wseg = [&](int t) {
                    float df = 1.f;
                    if constexpr (XSCALE) df = sDtf[t];
                    return (sSeg[t] == j) ? fast_exp2((float)(ce - sCum[t])) * df : 0.f;
                };
                // (cumulative decays restart at every segment in such a block)
                const float carry = fast_exp2((float)sCum[e]);
                f32x4 F[MTH];
                if (j == 0) {
#pragma unroll
                    for (int q = 0; q < MTH; ++q) F[q] = st[q] * carry;
                } else if (prm.init) {
                    const float* src = prm.init + (((int64_t)sSeqOf[j] * H + h) * P + p0 + lr) * N;
#pragma unroll
                    for (int q = 0; q < MTH; ++q) {
                        const float4 iv = *(const float4*)(src + nrow<N>(mb + q, 4 * lg));
                        F[q] = f32x4{iv.x, iv.y, iv.z, iv.w} * carry;
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < MTH; ++q) F[q] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    auto keep = [&](int t) { return sSeg[t] == j; };
                    const frag xw = mask_frag(weighted_x_frag<K::SWX>(sXr, LR, ks * KSTEP, xc, lr, lg, wseg),
                                              ks * KSTEP, lg, keep);
#pragma unroll
                    for (int q = 0; q < MTH; ++q)
                        F[q] = MF::mma(mask_frag(bt_frag<N, LB, K::SWB>(sB, mb + q, ks * KSTEP, lr, lg), ks * KSTEP, lg, keep),
                                       xw, F[q]);
                }
                if (j < nstart) {
                    if constexpr (!LOCAL) write_state(F, sSeqOf[j]);
                } else {
#pragma unroll
                    for (int q = 0; q < MTH; ++q) st[q] = F[q];
                }
            }
            // Settle this rare path's own memory traffic here, so that the
            // common path's wait counts stay exact (prefetches stay in flight).
            __builtin_amdgcn_s_waitcnt(0);
        }
    };

    // diagonal block (L o CB) X of this wave's token tiles, as X^T (L o CB)^T (token
    // tile r only needs s < 16 (r + 1)), then y = read-out + diagonal block + D x:
    // lane holds y[t = 16r + lr][p0 + 4lg .. +3], one 16-byte store per token tile
    // (past-the-end tokens are dropped by the range check).  Everything read from
    // X (the skip term and the X operands) is taken before the barrier that ends
    // the MFMA phase, so the next block's X may be staged right after it.
    auto diag_pre = [&]() {
        if (prm.D) {                                             // skip term (none without D)
#pragma unroll
            for (int i = 0; i < RTH; ++i) {
                const int t = 16 * K::own_tile(nh, i) + lr;
                float xv[4];
                if constexpr (SZ == 2) {
                    const bf16x4 x4 = *(const bf16x4*)(K::SWX ? sXr + unit_off<true>(t, (xc >> 2) + lg, LR)
                                                               : sXr + t * LR + xc + 4 * lg);
#pragma unroll
                    for (int q = 0; q < 4; ++q) xv[q] = (float)x4[q];
                } else {
                    const float4 x4 = *(const float4*)(sXr + t * LR + xc + 4 * lg);
                    xv[0] = x4.x; xv[1] = x4.y; xv[2] = x4.z; xv[3] = x4.w;
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[i][q] += Dh * xv[q];
            }
        }
        if constexpr (DKS > 0 && !XD_SHARED) {
#pragma unroll
            for (int q = 0; q < DKS; ++q) xd[q] = x_frag<K::SWX>(sXr, LR, 32 * q, xc, lr, lg);
        }
    };
    auto diag_phase = [&](int blk) {
        bool seg_done = false;
        if constexpr (SEQ) {
            if (nstart_c > 0) {
                // A block with sequence starts: one pass per segment, with the other
                // segments' X rows selected to zero and the result added to the
                // segment's own tokens only (L o CB is already zero across segments,
                // but zero times an Inf or NaN of another sequence would not be).
                for (int j = 0; j <= nstart_c; ++j) {
                    auto keep = [&](int t) { return sSeg[t] == j; };
#pragma unroll
                    for (int i = 0; i < RTH; ++i) {
                        const int r = K::own_tile(nh, i);
                        const TI* lrow = sLm + (16 * r + lr) * LQ + KPL * lg;
                        f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
                        if constexpr (DKS > 0) {
#pragma unroll
                            for (int q = 0; q < (i == 0 ? 1 : 2); ++q)
                                part = MF::mma(mask_frag(xd[q], 32 * q, lg, keep), lds_frag<TI>(lrow + 32 * q), part);
                        } else {
                            for (int ks = 0; ks < 16 * (r + 1); ks += KSTEP)
                                part = MF::mma(mask_frag(x_frag<K::SWX>(sXr, LR, ks, xc, lr, lg), ks, lg, keep),
                                               lds_frag<TI>(lrow + ks), part);
                        }
                        const bool in = sSeg[16 * r + lr] == j;
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[i][q] += in ? part[q] : 0.f;
                    }
                }
                seg_done = true;
            }
        }
        if (!seg_done) {
#pragma unroll
            for (int i = 0; i < RTH; ++i) {
                const int r = K::own_tile(nh, i);
                const TI* lrow = sLm + (16 * r + lr) * LQ + KPL * lg;
                if constexpr (DKS > 0) {
                    // tiles {0, 3} or {1, 2} (or {0} / {1}): one K step for the first, two for the second
#pragma unroll
                    for (int q = 0; q < (i == 0 ? 1 : 2); ++q) acc[i] = MF::mma(xd[q], lds_frag<TI>(lrow + 32 * q), acc[i]);
                } else {
                    for (int ks = 0; ks < 16 * (r + 1); ks += KSTEP)
                        acc[i] = MF::mma(x_frag<K::SWX>(sXr, LR, ks, xc, lr, lg), lds_frag<TI>(lrow + ks), acc[i]);
                }
            }
        }
        const int64_t t0 = (int64_t)blk * QB;
        const rsrc_t ry = make_rsrc(yrow + t0 * ys, yrec - t0 * ys);
#pragma unroll
        for (int i = 0; i < RTH; ++i) buf_store16<kYStorePolicy>(acc[i], ry, (16 * K::own_tile(nh, i) + lr) * ys + (xc + 4 * lg) * 4);
        if constexpr (SEQ) prevseq = lastseq_c;
    };

    if constexpr (!LOCAL) sx_store();    // the initial state, for the first read-out
    if (blk1 > blk0) {
        issue_bc(blk0);
        issue_x(blk0);
        prep(blk0);
    }
    block_sync_lds();
    // The initial state (loaded at entry) is carried through the loop; settle
    // its loads here so the loop header does not wait on memory each iteration.
    __builtin_amdgcn_s_waitcnt(0);
    for (int blk = blk0; blk < blk1; ++blk) {
        if (blk + 1 < blk1) issue_bc(blk + 1);
        if constexpr (!LOCAL) lm_phase();
        if (blk + 1 < blk1) issue_x(blk + 1);
        state_phase();
        if constexpr (!LOCAL) {
            lm_store();
            diag_pre();
        }
        // every wave's tiles of L o CB are written; the exchange area and block blk's
        // C, B, X and weighted X are no longer read (f32 without paired halves still
        // reads X in the diagonal product: it keeps a barrier before the next staging)
        block_sync_lds();
        if constexpr (!LOCAL) {
            sx_store();
            diag_phase(blk);
        } else if constexpr (SEQ) {
            prevseq = lastseq_c;
        }
        if (blk + 1 < blk1) {
            if constexpr (DKS == 0 && !LOCAL) block_sync_lds();
            prep(blk + 1);
            block_sync_lds();        // block blk+1's tiles (and the exchanged state) are complete
        }
    }
    if constexpr (LOCAL) {
        // this segment's end state from a zero incoming state, and the decay it
        // applies to an incoming state (none past a sequence start)
        float* dst = prm.seg_state + (slot * P + p0 + lr) * N;
#pragma unroll
        for (int j = 0; j < MTH; ++j)
            *(float4*)(dst + nrow<N>(mb + j, 4 * lg)) = make_float4(st[j][0], st[j][1], st[j][2], st[j][3]);
        if (head_leader && lane == 0) prm.seg_carry[slot] = seg_reset ? 0.f : fast_exp2((float)seg_total);
    } else if (sg == prm.nseg - 1) {
        // the state after the row's last token belongs to its last sequence
        if (T > 0 || !SEQ) write_state(st, prevseq);
    }
}

}  // namespace ssd
