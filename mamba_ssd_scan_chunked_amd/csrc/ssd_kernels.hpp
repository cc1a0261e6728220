// SSD chunked-scan forward kernels for gfx950 (MI355X).
//
// Two kernels make one forward pass:
//
//  1. ssd_prep_kernel, one workgroup per (row, group, block of QB tokens):
//       CB[t][s] = C_t . B_s   for t, s in the block (fp32), and B^T of the block.
//     These depend only on B and C, so every head of the group reuses them;
//     they are the intra-chunk C B^T products of the dual form Y = [L o (C B^T)] X
//     ("088 Mamba-2", section 2.2; the diagonal-block step of key design 2 on
//     the "Mamba-2 - Transformer and SSM share one algebra" page).
//
//  2. ssd_scan_kernel, one workgroup per (row, head), P/16 waves; wave w owns
//     channels p in [16w, 16w+16).  The workgroup walks its row block by block
//     (QB = 32 or 64 tokens) with the P x N state held in MFMA accumulator
//     registers for the whole row.  Per block:
//       a. log-decay l_t = dt_t A_h (kept in log2 units) and its inclusive
//          cumulative sum within the block, by a wavefront scan
//          (the within-chunk cumsum of the chunked algorithm);
//       b. masked decay L[t][s] = exp(cum_t - cum_s) for s <= t in the same
//          sequence, else 0, multiplied into CB (segment sum, section 2.2);
//       c. y_diag = (L o CB) X on bf16 MFMA (diagonal block, section 2.3);
//       d. y_off  = exp(cum_t) C_t H_prev, the incoming state read out by C and
//          decayed to each position (left factor, section 3 of "088 Mamba-2");
//       e. H <- exp(cum_end) H + X^T (exp(cum_end - cum_s) o B), the block's end
//          state combined with the carried one (right factor and the
//          inter-chunk scan step real_end = block_decay * prev + local_end);
//       f. y = y_off + y_diag + D x, written once to HBM in fp32.
//     Sequence boundaries inside a block (seq_idx) split it into segments:
//     L is masked across segments, each segment's incoming state is either the
//     carried state or its own initial state, and the state of a sequence that
//     ends inside the block is written to final_state on the spot.
//
// Because the state stays in registers, x is read once and y written once;
// the only other traffic is dt and the per-block CB / B^T tiles, which all
// heads of a group share through L2.

#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

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

// Number of K steps of the y_off product (K = N, permuted so that the state
// accumulators feed the B operand directly; see state_frags).
template <typename TI, int N> struct OffK {
    static constexpr int NK = N / Mfma<TI>::KSTEP;
};

// B-operand fragments of y_off = C . S^T built from the state accumulators.
// st[m] holds S^T rows n = 16m + 4*(l/16) + i.  bf16: step k packs tiles 2k and
// 2k+1 (n = 32k + 16*(e/4) + 4*(l/16) + e%4); fp32: step k = 4m + i.
template <int N>
__device__ inline void state_frags(const f32x4 (&st)[N / 16], bf16x8 (&sf)[N / 32]) {
#pragma unroll
    for (int k = 0; k < N / 32; ++k) {
        bf16x8 f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[i] = (__bf16)st[2 * k][i];
            f[4 + i] = (__bf16)st[2 * k + 1][i];
        }
        sf[k] = f;
    }
}
template <int N>
__device__ inline void state_frags(const f32x4 (&st)[N / 16], float (&sf)[N / 4]) {
#pragma unroll
    for (int m = 0; m < N / 16; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) sf[4 * m + i] = st[m][i];
}

// Same fragments from an fp32 state in global memory laid out [p][n] (row p = this lane's channel).
template <int N>
__device__ inline void global_state_frags(const float* row, int lg, bf16x8 (&sf)[N / 32]) {
#pragma unroll
    for (int k = 0; k < N / 32; ++k) {
        const float4 lo = *(const float4*)(row + 32 * k + 4 * lg);
        const float4 hi = *(const float4*)(row + 32 * k + 16 + 4 * lg);
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
        const float4 v = *(const float4*)(row + 16 * m + 4 * lg);
        sf[4 * m + 0] = v.x; sf[4 * m + 1] = v.y; sf[4 * m + 2] = v.z; sf[4 * m + 3] = v.w;
    }
}

// A-operand fragment of y_off: row t of the C tile at the permuted K indices.
__device__ inline bf16x8 c_frag(const __bf16* row, int k, int lg) {
    const bf16x4 lo = *(const bf16x4*)(row + 32 * k + 4 * lg);
    const bf16x4 hi = *(const bf16x4*)(row + 32 * k + 16 + 4 * lg);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ inline float c_frag(const float* row, int k, int lg) {
    return row[16 * (k >> 2) + 4 * lg + (k & 3)];
}

struct PrepParams {
    const void* B;
    const void* C;
    float* cb;          // (b, G, nblk, QB, QB) fp32
    void* bt;           // (b, G, nblk, N, QB) input dtype
    int64_t T, G;
    int nblk;
};

struct ScanParams {
    const void* x;
    const float* dt;
    const float* A_log;
    const float* D;
    const float* init;
    const int32_t* seq_idx;
    float* y;
    float* fin;
    const float* cb;
    const void* bt;
    const void* C;
    int64_t batch, T, H, G, nseqs;
    int nblk;
    int dt_scales_x;
};

// ============================================================== prep kernel
template <typename TI, int N, int QB>
__global__ __launch_bounds__(256) void ssd_prep_kernel(PrepParams prm) {
    constexpr int VE = 16 / sizeof(TI);         // elements per 16-byte vector
    constexpr int LP = N + VE;                  // padded row pitch (elements)
    __shared__ __attribute__((aligned(16))) TI sB[QB * LP];
    __shared__ __attribute__((aligned(16))) TI sC[QB * LP];

    const int tid = threadIdx.x;
    const int blk = blockIdx.x % prm.nblk;
    const int64_t bg = blockIdx.x / prm.nblk;   // b * G + g
    const int64_t b = bg / prm.G, g = bg % prm.G;
    const int64_t t0 = (int64_t)blk * QB;
    const int rows = (int)min((int64_t)QB, prm.T - t0);

    const TI* Bg = (const TI*)prm.B;
    const TI* Cg = (const TI*)prm.C;
    for (int v = tid; v < QB * N / VE; v += 256) {
        const int t = v / (N / VE), c = v % (N / VE);
        uint4 bv = make_uint4(0, 0, 0, 0), cv = make_uint4(0, 0, 0, 0);
        if (t < rows) {
            const int64_t off = ((b * prm.T + t0 + t) * prm.G + g) * N + c * VE;
            bv = *(const uint4*)(Bg + off);
            cv = *(const uint4*)(Cg + off);
        }
        *(uint4*)(sB + t * LP + c * VE) = bv;
        *(uint4*)(sC + t * LP + c * VE) = cv;
    }
    __syncthreads();

    // CB = C B^T over the block, 4x4 outputs per thread.
    constexpr int G4 = QB / 4;
    if (tid < G4 * G4) {
        const int tg = tid / G4, sg = tid % G4;
        float acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
        for (int n = 0; n < N; ++n) {
            float cv[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cv[i] = to_f32(sC[(4 * tg + i) * LP + n]);
                bv[i] = to_f32(sB[(4 * sg + i) * LP + n]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(cv[i], bv[j], acc[i][j]);
        }
        float* out = prm.cb + ((bg * prm.nblk + blk) * QB) * QB;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *(float4*)(out + (4 * tg + i) * QB + 4 * sg) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    }
    // B^T of the block (rows n, columns s), in the input dtype.
    TI* bt = (TI*)prm.bt + ((bg * prm.nblk + blk) * N) * QB;
    for (int v = tid; v < N * QB; v += 256) {
        const int n = v / QB, s = v % QB;
        bt[v] = sB[s * LP + n];
    }
}

// ============================================================== scan kernel
template <typename TI> struct CumType { typedef float type; };
template <> struct CumType<float> { typedef double type; };   // fp32 path: exponent differences in fp64

template <typename TI, int P, int N, int QB>
__global__ __launch_bounds__(P / 16 * 64) void ssd_scan_kernel(ScanParams prm) {
    typedef Mfma<TI> MF;
    typedef typename MF::frag frag;
    typedef typename CumType<TI>::type cum_t;
    constexpr int NW = P / 16;
    constexpr int NT = NW * 64;
    constexpr int VE = 16 / sizeof(TI);
    constexpr int LC = N + VE;      // sC pitch
    constexpr int LQ = QB + VE;     // pitch of rows indexed by s
    constexpr int KPL = MF::KPL, KSTEP = MF::KSTEP;
    constexpr int NK = OffK<TI, N>::NK;
    constexpr int RT = QB / 16;     // row tiles per block
    constexpr int MT = N / 16;      // state tiles per wave
    static_assert(QB <= 64 && QB % KSTEP == 0, "block length");
    static_assert(N % KSTEP == 0 && N % 16 == 0 && P % 16 == 0, "shape");

    __shared__ __attribute__((aligned(16))) TI sC[QB * LC];
    __shared__ __attribute__((aligned(16))) TI sBt[N * LQ];
    __shared__ __attribute__((aligned(16))) TI sLm[QB * LQ];
    __shared__ __attribute__((aligned(16))) TI sXt[P * LQ];
    __shared__ __attribute__((aligned(16))) TI sXw[P * LQ];
    __shared__ cum_t sCum[QB];
    __shared__ float sRow[QB];
    __shared__ float sDtf[QB];      // dt_s if x is scaled by dt, else 1
    __shared__ int sSeg[QB];
    __shared__ int sStart[QB + 1];
    __shared__ int sSeqOf[QB + 1];
    __shared__ int sNstart;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // Work-item order: runs of consecutive (row, head) items go to the same
    // XCD (workgroups are dealt round-robin over the 8 XCDs), so the heads of
    // a row share that row's CB / B^T tiles in one L2.
    const int64_t units = prm.batch * prm.H;
    int64_t u = blockIdx.x;
    if (units % 8 == 0) u = (int64_t)(blockIdx.x % 8) * (units / 8) + blockIdx.x / 8;
    const int64_t b = u / prm.H, h = u % prm.H;
    const int64_t g = h / (prm.H / prm.G);
    const int64_t T = prm.T, H = prm.H;
    const int p0 = 16 * w;

    // A_h in log2 units, so that the decays are exp2 of a cumulative sum
    cum_t A2;
    if constexpr (sizeof(cum_t) == 8) A2 = -exp((double)prm.A_log[h]) * 1.4426950408889634;
    else A2 = -expf(prm.A_log[h]) * 1.4426950408889634f;
    const float Dh = prm.D ? prm.D[h] : 0.f;
    const TI* xg = (const TI*)prm.x;
    const TI* btg = (const TI*)prm.bt;
    const int32_t* seqg = prm.seq_idx ? prm.seq_idx + b * T : nullptr;
    auto clamp_seq = [&](int s) { return s < 0 ? 0 : (s >= prm.nseqs ? (int)prm.nseqs - 1 : s); };

    // ---- initial state of the row's first sequence
    int prevseq = (int)b;
    if (seqg && T > 0) prevseq = clamp_seq(seqg[0]);
    f32x4 st[MT];
    if (prm.init) {
        const float* src = prm.init + (((int64_t)prevseq * H + h) * P + p0 + lr) * N;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float4 v = *(const float4*)(src + 16 * m + 4 * lg);
            st[m] = f32x4{v.x, v.y, v.z, v.w};
        }
    } else {
#pragma unroll
        for (int m = 0; m < MT; ++m) st[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    auto write_state = [&](const f32x4 (&s)[MT], int seq) {
        if (!prm.fin) return;
        float* dst = prm.fin + (((int64_t)seq * H + h) * P + p0 + lr) * N;
#pragma unroll
        for (int m = 0; m < MT; ++m)
            *(float4*)(dst + 16 * m + 4 * lg) = make_float4(s[m][0], s[m][1], s[m][2], s[m][3]);
    };

    for (int blk = 0; blk < prm.nblk; ++blk) {
        const int64_t t0 = (int64_t)blk * QB;
        const int rows = (int)min((int64_t)QB, T - t0);

        __syncthreads();   // the previous block's LDS contents are no longer read

        // ---- stage the C tile and the block's B^T tile
        {
            const TI* Cg = (const TI*)prm.C;
            for (int v = tid; v < QB * (N / VE); v += NT) {
                const int t = v / (N / VE), c = v % (N / VE);
                uint4 cv = make_uint4(0, 0, 0, 0);
                if (t < rows) cv = *(const uint4*)(Cg + ((b * T + t0 + t) * prm.G + g) * N + c * VE);
                *(uint4*)(sC + t * LC + c * VE) = cv;
            }
            const TI* btb = btg + (((b * prm.G + g) * prm.nblk + blk) * N) * QB;
            for (int v = tid; v < N * (QB / VE); v += NT) {
                const int n = v / (QB / VE), c = v % (QB / VE);
                *(uint4*)(sBt + n * LQ + c * VE) = *(const uint4*)(btb + n * QB + c * VE);
            }
        }
        // ---- X tile, stored transposed (rows p, columns t); raw vectors kept
        //      in registers for the weighted copy
        constexpr int XV = QB * (P / VE);
        constexpr int XPT = (XV + NT - 1) / NT;
        uint4 xr[XPT];
#pragma unroll
        for (int j = 0; j < XPT; ++j) {
            const int v = tid + j * NT;
            xr[j] = make_uint4(0, 0, 0, 0);
            if (v < XV) {
                const int t = v / (P / VE), c = v % (P / VE);
                if (t < rows) xr[j] = *(const uint4*)(xg + ((b * T + t0 + t) * H + h) * P + c * VE);
                const TI* e = (const TI*)&xr[j];
#pragma unroll
                for (int q = 0; q < VE; ++q) sXt[(c * VE + q) * LQ + t] = e[q];
            }
        }

        // ---- per-token scalars (wave 0, lane t = token t of the block):
        //      cumulative log2 decay, sequence segments
        if (w == 0) {
            const int t = lane;
            const bool valid = t < rows;
            float dtv = 0.f;
            int sq = prevseq;
            if (valid) {
                dtv = prm.dt[(b * T + t0 + t) * H + h];
                if (seqg) sq = clamp_seq(seqg[t0 + t]);
            } else if (seqg && rows > 0) {
                sq = clamp_seq(seqg[t0 + rows - 1]);
            }
            cum_t c = (cum_t)dtv * A2;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const cum_t o = __shfl_up(c, d);
                if (lane >= d) c += o;
            }
            const int up = __shfl_up(sq, 1);
            const int prev = (lane == 0) ? prevseq : up;
            const bool start = valid && (sq != prev);
            const uint64_t mask = __ballot(start);
            const uint64_t upto = (lane == 63) ? ~0ull : ((2ull << lane) - 1ull);
            const int seg = __popcll(mask & upto);
            if (t < QB) {
                sCum[t] = c;
                sSeg[t] = seg;
                sDtf[t] = prm.dt_scales_x ? dtv : 1.f;
            }
            if (start) {
                sStart[seg] = t;
                sSeqOf[seg] = sq;
            }
            if (lane == 0) {
                sStart[0] = 0;
                sSeqOf[0] = prevseq;
                sNstart = __popcll(mask);
            }
        }
        __syncthreads();

        const int nstart = sNstart;
        const int lastseq = sSeqOf[nstart];
        const cum_t cend = sCum[QB - 1];

        // ---- row scales of the incoming-state read-out: exp(cum_t - cum before t's segment)
        if (tid < QB) {
            const int a = sStart[sSeg[tid]];
            const cum_t before = (a == 0) ? (cum_t)0 : sCum[a - 1];
            sRow[tid] = fast_exp2((float)(sCum[tid] - before));
        }
        // ---- masked decay times C B^T:  Lm[t][s] = exp(cum_t - cum_s) CB[t][s]  (s <= t, same segment)
        {
            const float* cbb = prm.cb + (((b * prm.G + g) * prm.nblk + blk) * QB) * QB;
            for (int v = tid; v < QB * QB / 4; v += NT) {
                const int t = v / (QB / 4), s4 = (v % (QB / 4)) * 4;
                const float4 cv = *(const float4*)(cbb + t * QB + s4);
                const float cvals[4] = {cv.x, cv.y, cv.z, cv.w};
                const cum_t ct = sCum[t];
                const int segt = sSeg[t];
                TI out[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int s = s4 + q;
                    float lv = 0.f;
                    if (s <= t && sSeg[s] == segt) lv = fast_exp2((float)(ct - sCum[s])) * cvals[q] * sDtf[s];
                    out[q] = to_in<TI>(lv);
                }
                if constexpr (sizeof(TI) == 2) {
                    *(bf16x4*)(sLm + t * LQ + s4) = bf16x4{out[0], out[1], out[2], out[3]};
                } else {
                    *(float4*)(sLm + t * LQ + s4) = make_float4(out[0], out[1], out[2], out[3]);
                }
            }
        }
        // ---- weighted X for the end state: exp(cum_end - cum_s) x_s   (single-segment blocks)
        if (nstart == 0) {
#pragma unroll
            for (int j = 0; j < XPT; ++j) {
                const int v = tid + j * NT;
                if (v < XV) {
                    const int t = v / (P / VE), c = v % (P / VE);
                    const float ws = fast_exp2((float)(cend - sCum[t])) * sDtf[t];
                    const TI* e = (const TI*)&xr[j];
#pragma unroll
                    for (int q = 0; q < VE; ++q) sXw[(c * VE + q) * LQ + t] = to_in<TI>(ws * to_f32(e[q]));
                }
            }
        }
        __syncthreads();

        // ---- MFMA phase (wave w: channels p0 .. p0+15)
        frag sf[NK];
        state_frags<N>(st, sf);
        f32x4 acc_y[RT], acc_o[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            acc_y[r] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc_o[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // diagonal block (L o CB) X, causal: row tile r needs s < 16 (r + 1)
#pragma unroll
        for (int r = 0; r < RT; ++r) {
#pragma unroll
            for (int ks = 0; ks < 16 * (r + 1); ks += KSTEP) {
                const frag a = lds_frag<TI>(sLm + (16 * r + lr) * LQ + ks + KPL * lg);
                const frag bb = lds_frag<TI>(sXt + (p0 + lr) * LQ + ks + KPL * lg);
                acc_y[r] = MF::mma(a, bb, acc_y[r]);
            }
        }
        if (nstart == 0) {
            // incoming state read out by C
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int k = 0; k < NK; ++k)
                    acc_o[r] = MF::mma(c_frag(sC + (16 * r + lr) * LC, k, lg), sf[k], acc_o[r]);
            // carried state decayed over the block plus the block's own end state
            const float alpha = fast_exp2((float)cend);
#pragma unroll
            for (int m = 0; m < MT; ++m) st[m] *= alpha;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int ks = 0; ks < QB; ks += KSTEP) {
                    const frag a = lds_frag<TI>(sBt + (16 * m + lr) * LQ + ks + KPL * lg);
                    const frag bb = lds_frag<TI>(sXw + (p0 + lr) * LQ + ks + KPL * lg);
                    st[m] = MF::mma(a, bb, st[m]);
                }
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc_o[r][i] *= sRow[16 * r + 4 * lg + i];
        } else {
            // ---- block with sequence starts: one segment at a time
            // (1) read-out of each segment's incoming state
            for (int j = 0; j <= nstart; ++j) {
                const int a = sStart[j];
                const int e = (j < nstart) ? sStart[j + 1] - 1 : QB - 1;
                if (e < a) continue;                         // empty first segment
                frag f[NK];
                if (j == 0) {
#pragma unroll
                    for (int k = 0; k < NK; ++k) f[k] = sf[k];
                } else if (prm.init) {
                    global_state_frags<N>(prm.init + (((int64_t)sSeqOf[j] * H + h) * P + p0 + lr) * N, lg, f);
                } else {
                    continue;                                // zero initial state reads out nothing
                }
                f32x4 tmp[RT];
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    tmp[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k = 0; k < NK; ++k)
                        tmp[r] = MF::mma(c_frag(sC + (16 * r + lr) * LC, k, lg), f[k], tmp[r]);
                }
#pragma unroll
                for (int r = 0; r < RT; ++r)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 16 * r + 4 * lg + i;
                        if (sSeg[t] == j) acc_o[r][i] += sRow[t] * tmp[r][i];
                    }
            }
            // (2) state at the end of each segment: a sequence that ends inside
            //     the block hands its state to final_state; the last segment's
            //     state is carried on.
            if (sStart[1] == 0) write_state(st, sSeqOf[0]);   // previous sequence ended with the previous block
            for (int j = 0; j <= nstart; ++j) {
                const int a = sStart[j];
                const int e = (j < nstart) ? sStart[j + 1] - 1 : QB - 1;
                if (e < a) continue;
                __syncthreads();                             // sXw of the previous segment is consumed
#pragma unroll
                for (int jx = 0; jx < XPT; ++jx) {
                    const int v = tid + jx * NT;
                    if (v < XV) {
                        const int t = v / (P / VE), c = v % (P / VE);
                        const float ws = (sSeg[t] == j) ? fast_exp2((float)(sCum[e] - sCum[t])) * sDtf[t] : 0.f;
                        const TI* ev = (const TI*)&xr[jx];
#pragma unroll
                        for (int q = 0; q < VE; ++q) sXw[(c * VE + q) * LQ + t] = to_in<TI>(ws * to_f32(ev[q]));
                    }
                }
                __syncthreads();
                const cum_t before = (a == 0) ? (cum_t)0 : sCum[a - 1];
                const float carry = fast_exp2((float)(sCum[e] - before));
                f32x4 F[MT];
                if (j == 0) {
#pragma unroll
                    for (int m = 0; m < MT; ++m) F[m] = st[m] * carry;
                } else if (prm.init) {
                    const float* src = prm.init + (((int64_t)sSeqOf[j] * H + h) * P + p0 + lr) * N;
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        const float4 v = *(const float4*)(src + 16 * m + 4 * lg);
                        F[m] = f32x4{v.x, v.y, v.z, v.w} * carry;
                    }
                } else {
#pragma unroll
                    for (int m = 0; m < MT; ++m) F[m] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int ks = 0; ks < QB; ks += KSTEP) {
                        const frag a2 = lds_frag<TI>(sBt + (16 * m + lr) * LQ + ks + KPL * lg);
                        const frag bb = lds_frag<TI>(sXw + (p0 + lr) * LQ + ks + KPL * lg);
                        F[m] = MF::mma(a2, bb, F[m]);
                    }
                if (j < nstart) {
                    write_state(F, sSeqOf[j]);
                } else {
#pragma unroll
                    for (int m = 0; m < MT; ++m) st[m] = F[m];
                }
            }
        }

        // ---- y = read-out + diagonal block + D x, one fp32 write per element
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * r + 4 * lg + i;
                if (t < rows) {
                    const float xv = to_f32(sXt[(p0 + lr) * LQ + t]);
                    prm.y[((b * T + t0 + t) * H + h) * P + p0 + lr] = acc_o[r][i] + acc_y[r][i] + Dh * xv;
                }
            }
        prevseq = lastseq;
    }
    // state after the row's last token belongs to its last sequence
    if (T > 0 || !seqg) write_state(st, prevseq);
}

}  // namespace ssd
