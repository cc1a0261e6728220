// SSD backward for gfx950 (MI355X): the gradients of L = <dy, y> + <dfinal, final>
// with respect to x, dt, dt_bias, A_log, B, C, D and the initial states.
//
// The pages give the forward map only.  The backward is the chain rule applied
// to the recurrence of "088 Mamba-2" (section 2.1), H_t = a_t H_{t-1} +
// f_t x_t B_t^T, y_t = H_t C_t + D x_t, evaluated block by block in the same
// dual form as the forward (sections 2.2 and 3 of that page: masked
// attention-like products inside a block, a carried state between blocks).
// With G_t = dL/dH_t:
//   G_t  = dy_t C_t^T + a_{t+1} G_{t+1}       (after the last token: dfinal)
//   dC_t = sum_heads H_t^T dy_t,   dB_t = sum_heads f_t G_t^T x_t
//   dx_t = f_t G_t B_t + D dy_t
//   dl_t = dL/dlog a_t = <G_t, a_t H_{t-1}>,   u_t = x_t . (G_t B_t) = dL/df_t
// Inside a block of tokens with incoming state H_in and incoming gradient
// K (= a G of the first token after the block), dl_t splits exactly into
//   sum over s >= t > r of Z[s][r]  +  sum over s >= t of qoff_s
//   + sum over r < t of roff_r  +  2^cend <K, H_in>,
// Z[s][r] = 2^(cum_s - cum_r) f_r (dy_s . x_r)(C_s . B_r),
// qoff_s = 2^cum_s dy_s . (H_in C_s),  roff_r = 2^(cend - cum_r) f_r x_r . (K B_r),
// so that no rounding error is carried from block to block (a running sum of
// per-token terms over the whole row would accumulate it).
//
// ssd_bwd_fwd_kernel walks each (row, head) forwards with H on chip and
// produces the head's dC contribution, qoff and each block's incoming state
// (kept for the inner product above); ssd_bwd_rev_kernel walks it backwards
// with G on chip (as K, the gradient that reaches the block from its right)
// and produces dx, the head's dB contribution, Z (from the C B^T and dy x^T
// tiles it forms anyway), roff, dl, ddt, the per-row partial sums of dA_log,
// ddt_bias and dD, and dinit = a_0 G_0.  The contributions of the
// heads of a group are summed by ssd_bwd_group_sum_kernel (not needed when each
// group has one head: then the passes write dB and dC directly), the per-row
// scalars by ssd_bwd_scalars_kernel.
//
// Per 64-token block (32 for fp32 inputs) of QB tokens, with cum_t the inclusive
// cumulative log2 decay inside the block and cend = cum_{QB-1}:
//   forward pass:  W[t][s] = (s <= t) 2^(cum_t - cum_s) f_s (dy_t . x_s)
//                  dC^h   = W B + 2^cum_t dy H_in          (QB x N)
//                  H_out  = 2^cend H_in + X^T diag(f 2^(cend - cum)) B
//   reverse pass:  E[t][s] = (s >= t) 2^(cum_s - cum_t) (B_t . C_s)
//                  F[t][s] = (s >= t) 2^(cum_s - cum_t) (x_t . dy_s)
//                  GB      = E dY + 2^(cend - cum_t) B K^T  (QB x P; = G_t B_t)
//                  dB^h    = f_t (F C + 2^(cend - cum_t) X K)
//                  K_prev  = 2^cend K + dY^T diag(2^cum) C
// All products run on MFMA from tiles staged in LDS (bf16 operands with fp32
// accumulation for bf16 inputs, fp32 throughout for fp32 inputs); every
// operand is read either along its rows or, through the LDS transpose read,
// along its columns, so each tile is stored once.

#pragma once
#include "ssd_kernels.hpp"

namespace ssd {

struct BwdParams {
    const void* x;
    const float* dt;        // (batch, H, T): the dt input transposed, token-contiguous per (row, head)
    const float* dt_bias;
    const float* A_log;
    const void* B;
    const void* C;
    const float* D;
    const float* init;
    const float* dy;
    const float* dfinal;
    float* dx;
    float* ddt;
    void* dBh;        // (batch, T, HB, N): per-head dB (HB = H), or dB itself (HB = G = H)
    void* dCh;        // same for dC
    int h_bf16;       // per-head contributions stored as bf16 (bf16 inputs, HB = H > G), else fp32
    float* dinit;     // (batch, H, P, N) or null
    float* q;         // (batch, H, T) workspace: qoff
    void* hin;        // (H, hin_blocks, P * N) workspace: each block's incoming state (input type), in
                      // the order the state tiles are held: tile, lane, 4 values
    float* part;      // (batch, H, 3) workspace: per-row sums for dA (natural A), ddt_bias, dD
    int64_t batch, T, H, G, HB;
    int nblk;                 // blocks per row
    int64_t hin_blocks;       // block slots per head in hin
    // Packed sequences: (row, first token, end token, first hin slot) of each
    // sequence, or null when every row is one sequence.  A workgroup walks one
    // (sequence, head), with its blocks aligned to the sequence's first token.
    const int64_t* seqtab;
    // Rows split into nseg segments of seg_tokens tokens (nseg = 1: whole rows).
    // Segment s > 0 starts from seg_state[(row, head, s - 1)] (the forward state
    // entering it) instead of init; segment s < nseg - 1 takes seg_grad[(row,
    // head, s)] (the gradient with respect to its end state) instead of dfinal;
    // only segment 0 writes dinit.
    int nseg;
    int64_t seg_tokens;
    const float* seg_state;   // (batch, H, nseg - 1, P, N)
    const float* seg_grad;    // (batch, H, nseg - 1, P, N)
    int dt_softplus, x_scale;
};

// The token range a workgroup walks: sequence kq of the packed rows, segment kq
// of the split rows, or row kq.  Values are clamped, so inconsistent sequence
// ids stay memory-safe.  seg: the segment's index in its row (0 without split rows).
struct ItemRange {
    int64_t b, s0, len, hslot;
    int seg;
};
template <int QB>
__device__ inline ItemRange item_range(const BwdParams& prm, int64_t kq) {
    ItemRange r;
    r.seg = 0;
    if (!prm.seqtab && prm.nseg > 1) {
        r.b = kq / prm.nseg;
        r.seg = (int)(kq % prm.nseg);
        r.s0 = min((int64_t)r.seg * prm.seg_tokens, prm.T);
        r.len = min(prm.seg_tokens, prm.T - r.s0);
        r.hslot = kq * (prm.seg_tokens / QB);
    } else if (!prm.seqtab) {
        r.b = kq;
        r.s0 = 0;
        r.len = prm.T;
        r.hslot = kq * prm.nblk;
    } else {
        // one entry per workgroup: kept in scalar registers, so that the buffer
        // resources built from it are uniform
        const int64_t* e = prm.seqtab + 4 * kq;
        auto uni = [](int64_t v) {
            const int lo = __builtin_amdgcn_readfirstlane((int)(v & 0xffffffff));
            const int hi = __builtin_amdgcn_readfirstlane((int)(v >> 32));
            return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
        };
        r.b = min(max(uni(e[0]), (int64_t)0), prm.batch - 1);
        r.s0 = min(max(uni(e[1]), (int64_t)0), prm.T);
        r.len = min(max(uni(e[2]) - r.s0, (int64_t)0), prm.T - r.s0);
        r.hslot = max(uni(e[3]), (int64_t)0);
        if (r.hslot + (r.len + QB - 1) / QB > prm.hin_blocks) r.len = 0;
    }
    return r;
}

// Fragment of an operand stored with K contiguous: row `row`, K values
// k0 + KPL*(l/16) .. (bf16: one 16-byte read; fp32: one value).
__device__ inline bf16x8 frag_k(const __bf16* base, int pitch, int row, int k0, int lg) {
    return *(const bf16x8*)(base + row * pitch + k0 + 8 * lg);
}
__device__ inline float frag_k(const float* base, int pitch, int row, int k0, int lg) {
    return base[row * pitch + k0 + lg];
}
// Fragment of an operand stored with its rows contiguous (layout [k][m]):
// row m0 + l%16, K values k0 + KPL*(l/16) ..  (bf16: two LDS transpose reads).
__device__ inline bf16x8 frag_t(const __bf16* base, int pitch, int m0, int k0, int lr, int lg) {
    return x_frag(base, pitch, k0, m0, lr, lg);
}
__device__ inline float frag_t(const float* base, int pitch, int m0, int k0, int lr, int lg) {
    return base[(k0 + lg) * pitch + m0 + lr];
}
// The same with K value k scaled by wk[k] (rounded once to the input type).
__device__ inline bf16x8 frag_t_w(const __bf16* base, int pitch, int m0, int k0, int lr, int lg, const float* wk) {
    const bf16x8 v = x_frag(base, pitch, k0, m0, lr, lg);
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)(wk[k0 + 8 * lg + e] * (float)v[e]);
    return r;
}
__device__ inline float frag_t_w(const float* base, int pitch, int m0, int k0, int lr, int lg, const float* wk) {
    return wk[k0 + lg] * base[(k0 + lg) * pitch + m0 + lr];
}

// Four consecutive values of one row (8 bytes for bf16, 16 for fp32), LDS or global.
__device__ inline void store4(__bf16* dst, float a, float b, float c, float d) {
    *(bf16x4*)dst = bf16x4{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
}
__device__ inline void store4(float* dst, float a, float b, float c, float d) {
    *(f32x4*)dst = f32x4{a, b, c, d};
}

__device__ inline void buf_store_f32(float v, rsrc_t r, int off) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), r, off, 0, 0);
}
__device__ inline void buf_store_bf16(float v, rsrc_t r, int off) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)v), r, off, 0, 0);
}
// Four consecutive values of a dB / dC output: fp32, or bf16 for per-head
// contributions of bf16 inputs.
__device__ inline void store_grad4(f32x4 v, rsrc_t r, int64_t elem, int as_bf16) {
    if (as_bf16) {
        const bf16x4 h = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        typedef unsigned int u2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, h), r, (int)(elem * 2), 0, 0);
    } else {
        buf_store16(v, r, (int)(elem * 4));
    }
}
// Four consecutive values of one LDS row as fp32.
__device__ inline f32x4 lds_load4(const __bf16* p) {
    const bf16x4 v = *(const bf16x4*)p;
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ inline f32x4 lds_load4(const float* p) { return *(const f32x4*)p; }
// Sums across lane rows with gfx950's lane-swap instructions (VALU, no LDS
// permute).  v_permlane16_swap trades the odd 16-lane rows of its first operand
// for the even rows of its second; v_permlane32_swap the upper 32 lanes of the
// first for the lower 32 of the second.  Swapping v with zero leaves v's even rows
// (resp. lower half) in the first result and its odd rows (resp. upper half) moved
// down in the second, zero elsewhere, so the two results add to
//   add_xor16_even: v[l] + v[l + 16] in rows 0 and 2 (lanes 0-15, 32-47),
//   add_xor32_low:  v[l] + v[l + 32] in lanes 0-31,
// and to 0 in the other lanes.  The second result passes through an empty asm
// statement: in a sum of the two results, the compiler's optimizer replaced the
// second by the first (and added the first to itself).
__device__ inline float add_swapped(unsigned a, unsigned b) {
    asm volatile("" : "+v"(b));
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
__device__ inline float add_xor16_even(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v), 0u, false, false);
    return add_swapped(r[0], r[1]);
}
__device__ inline float add_xor32_low(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), 0u, false, false);
    return add_swapped(r[0], r[1]);
}
// The value of lane L (a constant), in every lane.
template <int L>
__device__ inline float lane_value(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), L));
}
template <int L>
__device__ inline double lane_value(double v) {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const unsigned lo = __builtin_amdgcn_readlane((int)(unsigned)u, L), hi = __builtin_amdgcn_readlane((int)(unsigned)(u >> 32), L);
    return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}
// Sum over the four lane groups (lanes with equal l % 16), valid in lanes 0-15
// (lane group 0) only: (v[l] + v[l+16]) + (v[l+32] + v[l+48]).
__device__ inline float group4_sum_lg0(float v) { return add_xor32_low(add_xor16_even(v)); }

// Sum over the 16 lanes of each lane group (lanes with equal l/16), left in the
// group's last lane (DPP row shifts, as in the wavefront scan).
__device__ inline float row16_sum(float v) {
    v = dpp_add<0x111, 0xf>(v);   // row_shr:1
    v = dpp_add<0x112, 0xf>(v);   // row_shr:2
    v = dpp_add<0x114, 0xf>(v);   // row_shr:4
    v = dpp_add<0x118, 0xf>(v);   // row_shr:8
    return v;
}

// Waves per workgroup of each backward kernel.
template <typename TI, int P, int N, int QB>
struct BwdWaves {
    static constexpr int FWD = 16, REV = 8, KLOC = 8;
};

template <typename TI, int P, int N, int QB, int NW_ = 8>
struct BwdCfg {
    static constexpr int NW = NW_, NT = 64 * NW;
    static constexpr int SZ = sizeof(TI);
    static constexpr int KSTEP = Mfma<TI>::KSTEP;
    static constexpr int PAD = SZ == 2 ? 8 : 4;                 // keeps 16-byte aligned rows
    static constexpr int LP = P + PAD, LN = N + PAD, LQ = QB + PAD;
    static constexpr int QT = QB / 16, PT = P / 16, NTL = N / 16;
    static constexpr int T_QQ = (QT * QT + NW - 1) / NW;       // token x token tiles per wave
    static constexpr int T_QN = (QT * NTL + NW - 1) / NW;      // token x state tiles per wave
    static constexpr int T_QP = (QT * PT + NW - 1) / NW;       // token x channel tiles per wave
    static constexpr int T_NP = (NTL * PT + NW - 1) / NW;      // state tiles per wave
    static constexpr int XU = QB * P * SZ / 16;                // 16-byte chunks of x per block
    static constexpr int YU = QB * P * 4 / 16;                 // of dy (fp32)
    static constexpr int BU = QB * N * SZ / 16;                // of B or C
    static constexpr int XPT = (XU + NT - 1) / NT, YPT = (YU + NT - 1) / NT, BPT = (BU + NT - 1) / NT;
    static_assert(QB == 32 || QB == 64, "block");
    static_assert(P % 16 == 0 && N % 16 == 0 && P % KSTEP == 0 && N % KSTEP == 0 && QB % KSTEP == 0, "shape");
};

// Staging of one block: global loads into registers (issued a block ahead),
// then into LDS.  dy is converted to the input type for the products.
template <typename TI, int P, int N, int QB, int NW_>
struct BwdStage {
    using K = BwdCfg<TI, P, N, QB, NW_>;
    uint4 xr[K::XPT], yr[K::YPT], br[K::BPT], cr[K::BPT];

    __device__ inline void issue(const char* xrow, int64_t xrec, int xs, const char* yrow, int64_t yrec, int ys,
                                 const char* brow, const char* crow, int64_t brec, int bs, int64_t t0, int tid) {
        const rsrc_t rx = make_rsrc(xrow + t0 * xs, xrec - t0 * xs);
        const rsrc_t ry = make_rsrc(yrow + t0 * ys, yrec - t0 * ys);
        const rsrc_t rb = make_rsrc(brow + t0 * bs, brec - t0 * bs);
        const rsrc_t rc = make_rsrc(crow + t0 * bs, brec - t0 * bs);
        constexpr int XC = P * K::SZ / 16, YC = P / 4, BC = N * K::SZ / 16;
#pragma unroll
        for (int j = 0; j < K::XPT; ++j) {
            const int v = tid + j * K::NT;
            if (K::XU % K::NT == 0 || v < K::XU) xr[j] = buf_load16(rx, (v / XC) * xs + (v % XC) * 16);
        }
#pragma unroll
        for (int j = 0; j < K::YPT; ++j) {
            const int v = tid + j * K::NT;
            if (K::YU % K::NT == 0 || v < K::YU) yr[j] = buf_load16(ry, (v / YC) * ys + (v % YC) * 16);
        }
#pragma unroll
        for (int j = 0; j < K::BPT; ++j) {
            const int v = tid + j * K::NT;
            if (K::BU % K::NT == 0 || v < K::BU) {
                br[j] = buf_load16(rb, (v / BC) * bs + (v % BC) * 16);
                cr[j] = buf_load16(rc, (v / BC) * bs + (v % BC) * 16);
            }
        }
    }
    __device__ inline void store(TI* sX, TI* sDY, TI* sB, TI* sC, int tid) const {
        constexpr int XC = P * K::SZ / 16, YC = P / 4, BC = N * K::SZ / 16, VE = 16 / K::SZ;
#pragma unroll
        for (int j = 0; j < K::XPT; ++j) {
            const int v = tid + j * K::NT;
            if (K::XU % K::NT == 0 || v < K::XU) *(uint4*)(sX + (v / XC) * K::LP + (v % XC) * VE) = xr[j];
        }
#pragma unroll
        for (int j = 0; j < K::YPT; ++j) {
            const int v = tid + j * K::NT;
            if (K::YU % K::NT == 0 || v < K::YU) {
                const float4 f = __builtin_bit_cast(float4, yr[j]);
                store4(sDY + (v / YC) * K::LP + (v % YC) * 4, f.x, f.y, f.z, f.w);
            }
        }
#pragma unroll
        for (int j = 0; j < K::BPT; ++j) {
            const int v = tid + j * K::NT;
            if (K::BU % K::NT == 0 || v < K::BU) {
                *(uint4*)(sB + (v / BC) * K::LN + (v % BC) * VE) = br[j];
                *(uint4*)(sC + (v / BC) * K::LN + (v % BC) * VE) = cr[j];
            }
        }
    }
};

// ------------------------------------------------------------ forward pass
template <typename TI, int P, int N, int QB>
__global__ __launch_bounds__((64 * BwdWaves<TI, P, N, QB>::FWD)) void ssd_bwd_fwd_kernel(BwdParams prm) {
    using K = BwdCfg<TI, P, N, QB, BwdWaves<TI, P, N, QB>::FWD>;
    using M = Mfma<TI>;
    typedef typename CumType<TI>::type cum_t;
    constexpr int NW = K::NW, LP = K::LP, LN = K::LN, LQ = K::LQ, QT = K::QT, PT = K::PT, NTL = K::NTL;
    constexpr int KS = M::KSTEP;
    __shared__ __attribute__((aligned(16))) TI sDY[QB * LP];
    __shared__ __attribute__((aligned(16))) TI sX[QB * LP];
    __shared__ __attribute__((aligned(16))) TI sB[QB * LN];
    __shared__ __attribute__((aligned(16))) TI sC[QB * LN];
    __shared__ __attribute__((aligned(16))) TI sW[QB * LQ];
    __shared__ __attribute__((aligned(16))) TI sS[P * LN];    // carried state H[p][n], operand copy
    __shared__ __attribute__((aligned(16))) cum_t sCum[64];
    __shared__ __attribute__((aligned(16))) float sF[64];      // input factor f_s
    __shared__ __attribute__((aligned(16))) float sWx[64];     // f_s 2^(cend - cum_s)
    __shared__ __attribute__((aligned(16))) float sDin[64];    // 2^cum_t
    __shared__ float sQp[NTL][QB];
    __shared__ float sCend;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
    // item: (sequence or row kq, head h); tokens s0 .. s0+len-1 of row b
    const int64_t H = prm.H, G = prm.G, HB = prm.HB;
    const int64_t kq = blockIdx.x / H, h = blockIdx.x % H;
    const ItemRange ir = item_range<QB>(prm, kq);
    const int64_t b = ir.b, T = ir.len, tb = b * prm.T + ir.s0;   // T: this item's tokens; tb: its first token
    const int64_t bh = kq * H + h;          // (item, head): per-item sums
    const int64_t sh = prm.seqtab ? bh : b * H + h;   // (sequence or row, head): init, dfinal, dinit
    const int64_t rh = b * H + h;           // (row, head): the token-contiguous dt and qoff runs
    const int nblk = (int)((T + QB - 1) / QB);
    const int64_t g = h / (H / G), hb = HB == H ? h : g;
    // the state entering the item (forward pass), the gradient leaving its end (reverse
    // pass) and where dinit goes (null: none), each P x N fp32 or null for zero
    const int64_t PN = (int64_t)P * N;
    const int64_t slot = (b * H + h) * (prm.nseg - 1) + ir.seg;     // split rows: this segment's slot
    const float* item_init = ir.seg > 0 ? prm.seg_state + (slot - 1) * PN : (prm.init ? prm.init + sh * PN : nullptr);
    const float* item_dfinal = ir.seg < prm.nseg - 1 ? prm.seg_grad + slot * PN
                                                     : (prm.dfinal ? prm.dfinal + sh * PN : nullptr);
    float* item_dinit = ir.seg == 0 && prm.dinit ? prm.dinit + sh * PN : nullptr;
    (void)item_init; (void)item_dfinal; (void)item_dinit;
    constexpr int SZ = K::SZ;
    const int xs = (int)(H * P * SZ), ys = (int)(H * P * 4), bs = (int)(G * N * SZ);
    const char* xrow = (const char*)prm.x + (tb * H + h) * P * SZ;
    const char* yrow = (const char*)prm.dy + (tb * H + h) * P * 4;
    const char* brow = (const char*)prm.B + (tb * G + g) * N * SZ;
    const char* crow = (const char*)prm.C + (tb * G + g) * N * SZ;
    const int64_t xrec = T * xs, yrec = T * ys, brec = T * bs;
    const float Anat = -expf(prm.A_log[h]);
    cum_t A2;
    if constexpr (sizeof(cum_t) == 8) A2 = -exp((double)prm.A_log[h]) * 1.4426950408889634;
    else A2 = Anat * 1.4426950408889634f;
    const float dtb = prm.dt_bias ? prm.dt_bias[h] : 0.f;

    BwdStage<TI, P, N, QB, K::NW> stg;
    float dtn = 0.f;                      // wave 1: the next block's dt (lane = token)
    auto issue = [&](int blk) {
        const int64_t t0 = (int64_t)blk * QB;
        stg.issue(xrow, xrec, xs, yrow, yrec, ys, brow, crow, brec, bs, t0, tid);
        if (w == 1) dtn = buf_load_f32(make_rsrc(prm.dt + rh * prm.T + ir.s0 + t0, (T - t0) * 4), lane * 4);
    };
    // per-token scalars of a block (wave 1, lane = token)
    auto scalars = [&](int blk) {
        const int rows = (int)min((int64_t)QB, T - (int64_t)blk * QB);
        const float d = lane < rows ? step_size(dtn + dtb, prm.dt_softplus) : 0.f;
        const cum_t cum = wave_incl_scan((cum_t)d * A2);
        const cum_t cend = lane_value<QB - 1>(cum);
        const float f = x_factor(d, Anat, prm.x_scale);
        if (lane < QB) {
            sCum[lane] = cum;
            sF[lane] = f;
            sWx[lane] = f * fast_exp2((float)(cend - cum));
            sDin[lane] = fast_exp2((float)cum);
        }
        if (lane == 0) sCend = fast_exp2((float)cend);
    };

    // carried state H^T as accumulator tiles (rows n, columns p), and its operand copy
    f32x4 st[K::T_NP];
#pragma unroll
    for (int j = 0; j < K::T_NP; ++j) {
        const int tile = w + NW * j;
        st[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tile < NTL * PT) {
            const int n0 = 16 * (tile / PT) + 4 * lg, p = 16 * (tile % PT) + lr;
            if (item_init) {
                const float4 v = *(const float4*)(item_init + p * N + n0);
                st[j] = f32x4{v.x, v.y, v.z, v.w};
            }
            store4(sS + p * LN + n0, st[j][0], st[j][1], st[j][2], st[j][3]);
        }
    }

    if (nblk > 0) {                       // (uniform over the workgroup)
        issue(0);
        stg.store(sX, sDY, sB, sC, tid);
        if (w == 1) scalars(0);
        block_sync_lds();
    }

    for (int blk = 0; blk < nblk; ++blk) {
        const int64_t t0 = (int64_t)blk * QB;
        if (blk + 1 < nblk) issue(blk + 1);

        // ---- phase A: the incoming state to the workspace; W^T tiles (rows s, columns t), and dy H_in
        {
            TI* hb0 = (TI*)prm.hin + (h * prm.hin_blocks + ir.hslot + blk) * (int64_t)(P * N);
#pragma unroll
            for (int j = 0; j < K::T_NP; ++j) {
                const int tile = w + NW * j;
                if (tile < NTL * PT) store4(hb0 + (tile * 64 + lane) * 4, st[j][0], st[j][1], st[j][2], st[j][3]);
            }
        }
#pragma unroll
        for (int j = 0; j < K::T_QQ; ++j) {
            const int tile = w + NW * j;
            if (tile < QT * QT) {
                const int si = tile / QT, ti = tile % QT;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k0 = 0; k0 < P; k0 += KS)
                    acc = M::mma(frag_k(sX, LP, 16 * si + lr, k0, lg), frag_k(sDY, LP, 16 * ti + lr, k0, lg), acc);
                const int t = 16 * ti + lr, s0 = 16 * si + 4 * lg;
                const cum_t ct = sCum[t];
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = s0 + e;
                    v[e] = s <= t ? fast_exp2((float)(ct - sCum[s])) * sF[s] * acc[e] : 0.f;
                }
                store4(sW + t * LQ + s0, v[0], v[1], v[2], v[3]);
            }
        }
        f32x4 a3[K::T_QN];
#pragma unroll
        for (int j = 0; j < K::T_QN; ++j) {
            const int tile = w + NW * j;
            a3[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (tile < QT * NTL) {
                const int ti = tile / NTL, ni = tile % NTL;
#pragma unroll
                for (int k0 = 0; k0 < P; k0 += KS)
                    a3[j] = M::mma(frag_t(sS, LN, 16 * ni, k0, lr, lg), frag_k(sDY, LP, 16 * ti + lr, k0, lg), a3[j]);
            }
        }
        block_sync_lds();

        // ---- phase B: dC^h = W B + 2^cum dy H_in, q partial sums; state update
        {
            const int es = prm.h_bf16 ? 2 : 4;
            const rsrc_t rdc = make_rsrc((char*)prm.dCh + ((tb + t0) * HB + hb) * N * es, (T - t0) * HB * N * es);
#pragma unroll
            for (int j = 0; j < K::T_QN; ++j) {
                const int tile = w + NW * j;
                if (tile < QT * NTL) {
                    const int ti = tile / NTL, ni = tile % NTL;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k0 = 0; k0 < QB; k0 += KS)
                        acc = M::mma(frag_t(sB, LN, 16 * ni, k0, lr, lg), frag_k(sW, LQ, 16 * ti + lr, k0, lg), acc);
                    // this lane: state rows n0 .. n0+3 of token t
                    const int t = 16 * ti + lr, n0 = 16 * ni + 4 * lg;
                    const f32x4 off = a3[j] * sDin[t];
                    store_grad4(acc + off, rdc, t * HB * N + n0, prm.h_bf16);
                    const f32x4 c4 = lds_load4(sC + t * LN + n0);
                    const float qs = group4_sum_lg0(off[0] * c4[0] + off[1] * c4[1] + off[2] * c4[2] + off[3] * c4[3]);
                    if (lg == 0) sQp[ni][t] = qs;
                }
            }
            const float dec = sCend;
            // every state tile of this wave has channel tile w mod PT: its weighted X
            // operands are formed once for all of them
            static_assert(NW % PT == 0, "a wave's state tiles share one channel tile");
            decltype(frag_t_w(sX, LP, 0, 0, lr, lg, sWx)) xw[QB / KS];
#pragma unroll
            for (int k0 = 0; k0 < QB; k0 += KS) xw[k0 / KS] = frag_t_w(sX, LP, 16 * (w % PT), k0, lr, lg, sWx);
#pragma unroll
            for (int j = 0; j < K::T_NP; ++j) {
                const int tile = w + NW * j;
                if (tile < NTL * PT) {
                    const int ni = tile / PT, pj = tile % PT;
                    f32x4 acc = st[j] * dec;
#pragma unroll
                    for (int k0 = 0; k0 < QB; k0 += KS)
                        acc = M::mma(frag_t(sB, LN, 16 * ni, k0, lr, lg), xw[k0 / KS], acc);
                    st[j] = acc;
                    store4(sS + (16 * pj + lr) * LN + 16 * ni + 4 * lg, acc[0], acc[1], acc[2], acc[3]);
                }
            }
        }
        block_sync_lds();

        // ---- phase C: q (wave 0), then the next block into LDS and its scalars (wave 1)
        if (w == 0 && lane < QB) {
            float qv = 0.f;
#pragma unroll
            for (int ni = 0; ni < NTL; ++ni) qv += sQp[ni][lane];
            if (t0 + lane < T) prm.q[rh * prm.T + ir.s0 + t0 + lane] = qv;
        }
        if (blk + 1 < nblk) {
            stg.store(sX, sDY, sB, sC, tid);
            if (w == 1) scalars(blk + 1);
        }
        block_sync_lds();
    }

}

// ------------------------------------------------------------ reverse pass
template <typename TI, int P, int N, int QB>
__global__ __launch_bounds__((64 * BwdWaves<TI, P, N, QB>::REV)) void ssd_bwd_rev_kernel(BwdParams prm) {
    using K = BwdCfg<TI, P, N, QB, BwdWaves<TI, P, N, QB>::REV>;
    using M = Mfma<TI>;
    typedef typename CumType<TI>::type cum_t;
    constexpr int NW = K::NW, LP = K::LP, LN = K::LN, LQ = K::LQ, QT = K::QT, PT = K::PT, NTL = K::NTL;
    constexpr int KS = M::KSTEP;
    __shared__ __attribute__((aligned(16))) TI sDY[QB * LP];
    __shared__ __attribute__((aligned(16))) TI sX[QB * LP];
    __shared__ __attribute__((aligned(16))) TI sB[QB * LN];
    __shared__ __attribute__((aligned(16))) TI sC[QB * LN];
    __shared__ __attribute__((aligned(16))) TI sE[QB * LQ];
    __shared__ __attribute__((aligned(16))) TI sFm[QB * LQ];
    __shared__ __attribute__((aligned(16))) TI sK[P * LN];    // K[p][n], operand copy
    __shared__ __attribute__((aligned(16))) cum_t sCum[64];
    __shared__ __attribute__((aligned(16))) float sF[64];      // f_t
    __shared__ __attribute__((aligned(16))) float sDin[64];    // 2^cum_t
    __shared__ __attribute__((aligned(16))) float sDout[64];   // 2^(cend - cum_t)
    __shared__ __attribute__((aligned(16))) float sDel[64];    // step size Delta_t
    __shared__ __attribute__((aligned(16))) float sPre[64];    // dt + bias (softplus argument)
    __shared__ float sUp[PT][QB];      // x . (G B) over each 16-channel tile
    __shared__ float sUop[PT][QB];     // x . (2^(cend - cum) K B) over each tile
    __shared__ float sDDp[PT][QB];     // x . dy over each tile
    __shared__ float sCz[QT][QB];      // column sums of Z below the diagonal, per row tile
    __shared__ float sRz[QT][QB];      // row sums of Z left of the diagonal, per column tile
    __shared__ float sKap[NW];         // <K, H_in> over each wave's state tiles
    __shared__ float sCend;

    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: per-wave branches stay scalar
    // item: (sequence or row kq, head h); tokens s0 .. s0+len-1 of row b
    const int64_t H = prm.H, G = prm.G, HB = prm.HB;
    const int64_t kq = blockIdx.x / H, h = blockIdx.x % H;
    const ItemRange ir = item_range<QB>(prm, kq);
    const int64_t b = ir.b, T = ir.len, tb = b * prm.T + ir.s0;   // T: this item's tokens; tb: its first token
    const int64_t bh = kq * H + h;          // (item, head): per-item sums
    const int64_t sh = prm.seqtab ? bh : b * H + h;   // (sequence or row, head): init, dfinal, dinit
    const int64_t rh = b * H + h;           // (row, head): the token-contiguous dt and qoff runs
    const int nblk = (int)((T + QB - 1) / QB);
    const int64_t g = h / (H / G), hb = HB == H ? h : g;
    // the state entering the item (forward pass), the gradient leaving its end (reverse
    // pass) and where dinit goes (null: none), each P x N fp32 or null for zero
    const int64_t PN = (int64_t)P * N;
    const int64_t slot = (b * H + h) * (prm.nseg - 1) + ir.seg;     // split rows: this segment's slot
    const float* item_init = ir.seg > 0 ? prm.seg_state + (slot - 1) * PN : (prm.init ? prm.init + sh * PN : nullptr);
    const float* item_dfinal = ir.seg < prm.nseg - 1 ? prm.seg_grad + slot * PN
                                                     : (prm.dfinal ? prm.dfinal + sh * PN : nullptr);
    float* item_dinit = ir.seg == 0 && prm.dinit ? prm.dinit + sh * PN : nullptr;
    (void)item_init; (void)item_dfinal; (void)item_dinit;
    constexpr int SZ = K::SZ;
    const int xs = (int)(H * P * SZ), ys = (int)(H * P * 4), bs = (int)(G * N * SZ);
    const char* xrow = (const char*)prm.x + (tb * H + h) * P * SZ;
    const char* yrow = (const char*)prm.dy + (tb * H + h) * P * 4;
    const char* brow = (const char*)prm.B + (tb * G + g) * N * SZ;
    const char* crow = (const char*)prm.C + (tb * G + g) * N * SZ;
    const int64_t xrec = T * xs, yrec = T * ys, brec = T * bs;
    const float Anat = -expf(prm.A_log[h]);
    cum_t A2;
    if constexpr (sizeof(cum_t) == 8) A2 = -exp((double)prm.A_log[h]) * 1.4426950408889634;
    else A2 = Anat * 1.4426950408889634f;
    const float dtb = prm.dt_bias ? prm.dt_bias[h] : 0.f;
    const float Dh = prm.D ? prm.D[h] : 0.f;

    BwdStage<TI, P, N, QB, K::NW> stg;
    // the next block's per-token input of waves 0 and 1 (lane = token): qoff for wave 0,
    // dt for wave 1.  One variable for both: with two, each assigned in its own wave's
    // branch, the compiler kept them in scratch memory behind a wait for every
    // outstanding load.
    float nxt = 0.f;
    // the block's incoming state at this lane's state-tile positions (4 values per tile)
    typedef typename std::conditional<K::SZ == 2, uint2, uint4>::type h4_t;
    // (no branch around the loads, so that nothing waits for them before their use)
    auto load_hin = [&](int blk, h4_t (&hv)[K::T_NP]) {
        const TI* hb0 = (const TI*)prm.hin + (h * prm.hin_blocks + ir.hslot + blk) * (int64_t)(P * N);
#pragma unroll
        for (int j = 0; j < K::T_NP; ++j) {
            const int tile = min(w + NW * j, NTL * PT - 1);      // surplus slots reload a valid tile
            hv[j] = *(const h4_t*)(hb0 + (tile * 64 + lane) * 4);
        }
    };
    auto issue = [&](int blk) {
        const int64_t t0 = (int64_t)blk * QB;
        stg.issue(xrow, xrec, xs, yrow, yrec, ys, brow, crow, brec, bs, t0, tid);
        if (w <= 1) {
            const float* src = w == 1 ? prm.dt : prm.q;
            nxt = buf_load_f32(make_rsrc(src + rh * prm.T + ir.s0 + t0, (T - t0) * 4), lane * 4);
        }
    };
    float qcur = 0.f;
    auto scalars = [&](int blk) {
        const int rows = (int)min((int64_t)QB, T - (int64_t)blk * QB);
        const float pre = nxt + dtb;          // (wave 1: nxt is dt)
        const float d = lane < rows ? step_size(pre, prm.dt_softplus) : 0.f;
        const cum_t cum = wave_incl_scan((cum_t)d * A2);
        const cum_t cend = lane_value<QB - 1>(cum);
        if (lane < QB) {
            sCum[lane] = cum;
            sF[lane] = x_factor(d, Anat, prm.x_scale);
            sDin[lane] = fast_exp2((float)cum);
            sDout[lane] = fast_exp2((float)(cend - cum));
            sDel[lane] = d;
            sPre[lane] = pre;
        }
        if (lane == 0) sCend = fast_exp2((float)cend);
    };

    // carried K^T = (a_{t+1} G_{t+1})^T as accumulator tiles (rows n, columns p)
    f32x4 kst[K::T_NP];
#pragma unroll
    for (int j = 0; j < K::T_NP; ++j) {
        const int tile = w + NW * j;
        kst[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tile < NTL * PT) {
            const int n0 = 16 * (tile / PT) + 4 * lg, p = 16 * (tile % PT) + lr;
            if (item_dfinal) {
                const float4 v = *(const float4*)(item_dfinal + p * N + n0);
                kst[j] = f32x4{v.x, v.y, v.z, v.w};
            }
            store4(sK + p * LN + n0, kst[j][0], kst[j][1], kst[j][2], kst[j][3]);
        }
    }

    // wave 0: per-row sums
    typedef cum_t acc_t;
    acc_t sum_dA = 0, sum_bias = 0, sum_D = 0;
    const int fdmode = prm.x_scale;

    if (nblk > 0) {                       // (uniform over the workgroup)
        issue(nblk - 1);
        stg.store(sX, sDY, sB, sC, tid);
        if (w == 1) scalars(nblk - 1);
        qcur = nxt;                       // (wave 0: nxt is qoff)
        block_sync_lds();
    }

    for (int blk = nblk - 1; blk >= 0; --blk) {
        const int64_t t0 = (int64_t)blk * QB;
        h4_t hcur[K::T_NP];
        load_hin(blk, hcur);              // used after this block's first products
        if (blk > 0) issue(blk - 1);

        // ---- phase A: E and F (from E^T, F^T tiles: rows s, columns t), B K^T, X K
#pragma unroll
        for (int j = 0; j < K::T_QQ; ++j) {
            const int tile = w + NW * j;
            if (tile < QT * QT) {
                const int si = tile / QT, ti = tile % QT;
                f32x4 ae = {0.f, 0.f, 0.f, 0.f}, af = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k0 = 0; k0 < N; k0 += KS)
                    ae = M::mma(frag_k(sC, LN, 16 * si + lr, k0, lg), frag_k(sB, LN, 16 * ti + lr, k0, lg), ae);
#pragma unroll
                for (int k0 = 0; k0 < P; k0 += KS)
                    af = M::mma(frag_k(sDY, LP, 16 * si + lr, k0, lg), frag_k(sX, LP, 16 * ti + lr, k0, lg), af);
                const int t = 16 * ti + lr, s0 = 16 * si + 4 * lg;
                const cum_t ct = sCum[t];
                const float ft = sF[t];
                float ve[4], vf[4], zc = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = s0 + e;
                    const float m = s >= t ? fast_exp2((float)(sCum[s] - ct)) : 0.f;
                    ve[e] = s >= t ? m * ae[e] : 0.f;
                    vf[e] = s >= t ? m * af[e] : 0.f;
                    // Z[s][t] below the diagonal: its column sum (over s) and row sum (over t)
                    const float z = s > t ? m * ft * ae[e] * af[e] : 0.f;
                    zc += z;
                    const float zr = row16_sum(z);
                    if (lr == 15) sRz[ti][s] = zr;
                }
                zc = group4_sum_lg0(zc);
                if (lg == 0) sCz[si][t] = zc;
                store4(sE + t * LQ + s0, ve[0], ve[1], ve[2], ve[3]);
                store4(sFm + t * LQ + s0, vf[0], vf[1], vf[2], vf[3]);
            }
        }
        f32x4 a3[K::T_QP];
#pragma unroll
        for (int j = 0; j < K::T_QP; ++j) {
            const int tile = w + NW * j;
            a3[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (tile < QT * PT) {
                const int ti = tile / PT, pj = tile % PT;
#pragma unroll
                for (int k0 = 0; k0 < N; k0 += KS)
                    a3[j] = M::mma(frag_k(sK, LN, 16 * pj + lr, k0, lg), frag_k(sB, LN, 16 * ti + lr, k0, lg), a3[j]);
            }
        }
        {   // <K, H_in> over this wave's state tiles (K as it enters the block)
            float kp = 0.f;
#pragma unroll
            for (int j = 0; j < K::T_NP; ++j) {
                const int tile = w + NW * j;
                if (tile < NTL * PT) {
                    const TI* hv = (const TI*)&hcur[j];
#pragma unroll
                    for (int e = 0; e < 4; ++e) kp += kst[j][e] * to_f32(hv[e]);
                }
            }
            kp = add_xor32_low(add_xor16_even(kp));          // lanes 0-15 hold the sums of their four lane groups
#pragma unroll
            for (int d = 8; d >= 1; d >>= 1) kp += __shfl_xor(kp, d);      // (within lanes 0-15)
            if (lane == 0) sKap[w] = kp;
        }
        f32x4 a5[K::T_QN];
#pragma unroll
        for (int j = 0; j < K::T_QN; ++j) {
            const int tile = w + NW * j;
            a5[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (tile < QT * NTL) {
                const int ti = tile / NTL, ni = tile % NTL;
#pragma unroll
                for (int k0 = 0; k0 < P; k0 += KS)
                    a5[j] = M::mma(frag_t(sK, LN, 16 * ni, k0, lr, lg), frag_k(sX, LP, 16 * ti + lr, k0, lg), a5[j]);
            }
        }
        block_sync_lds();

        // ---- phase B: G B (-> dx, u, dy.x), dB^h, K update
        {
            const rsrc_t rdx = make_rsrc(prm.dx + ((tb + t0) * H + h) * P, (T - t0) * H * P * 4);
#pragma unroll
            for (int j = 0; j < K::T_QP; ++j) {
                const int tile = w + NW * j;
                if (tile < QT * PT) {
                    const int ti = tile / PT, pj = tile % PT;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k0 = 0; k0 < QB; k0 += KS)
                        acc = M::mma(frag_t(sDY, LP, 16 * pj, k0, lr, lg), frag_k(sE, LQ, 16 * ti + lr, k0, lg), acc);
                    // this lane: channels p0 .. p0+3 of token t
                    const int t = 16 * ti + lr, p0 = 16 * pj + 4 * lg;
                    const f32x4 gof = a3[j] * sDout[t];
                    const f32x4 gb = acc + gof;
                    const f32x4 dy4 = lds_load4(sDY + t * LP + p0), x4 = lds_load4(sX + t * LP + p0);
                    buf_store16(gb * sF[t] + dy4 * Dh, rdx, (int)((t * H * P + p0) * 4));
                    const float us = group4_sum_lg0(x4[0] * gb[0] + x4[1] * gb[1] + x4[2] * gb[2] + x4[3] * gb[3]);
                    const float uo = group4_sum_lg0(x4[0] * gof[0] + x4[1] * gof[1] + x4[2] * gof[2] + x4[3] * gof[3]);
                    const float ds = group4_sum_lg0(x4[0] * dy4[0] + x4[1] * dy4[1] + x4[2] * dy4[2] + x4[3] * dy4[3]);
                    if (lg == 0) {
                        sUp[pj][t] = us;
                        sUop[pj][t] = uo;
                        sDDp[pj][t] = ds;
                    }
                }
            }
            const int es = prm.h_bf16 ? 2 : 4;
            const rsrc_t rdb = make_rsrc((char*)prm.dBh + ((tb + t0) * HB + hb) * N * es, (T - t0) * HB * N * es);
#pragma unroll
            for (int j = 0; j < K::T_QN; ++j) {
                const int tile = w + NW * j;
                if (tile < QT * NTL) {
                    const int ti = tile / NTL, ni = tile % NTL;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k0 = 0; k0 < QB; k0 += KS)
                        acc = M::mma(frag_t(sC, LN, 16 * ni, k0, lr, lg), frag_k(sFm, LQ, 16 * ti + lr, k0, lg), acc);
                    const int t = 16 * ti + lr, n0 = 16 * ni + 4 * lg;
                    store_grad4((acc + a5[j] * sDout[t]) * sF[t], rdb, t * HB * N + n0, prm.h_bf16);
                }
            }
            const float dec = sCend;
            // every state tile of this wave has channel tile w mod PT: its weighted dY
            // operands are formed once for all of them
            static_assert(NW % PT == 0, "a wave's state tiles share one channel tile");
            decltype(frag_t_w(sDY, LP, 0, 0, lr, lg, sDin)) yw[QB / KS];
#pragma unroll
            for (int k0 = 0; k0 < QB; k0 += KS) yw[k0 / KS] = frag_t_w(sDY, LP, 16 * (w % PT), k0, lr, lg, sDin);
#pragma unroll
            for (int j = 0; j < K::T_NP; ++j) {
                const int tile = w + NW * j;
                if (tile < NTL * PT) {
                    const int ni = tile / PT, pj = tile % PT;
                    f32x4 acc = kst[j] * dec;
#pragma unroll
                    for (int k0 = 0; k0 < QB; k0 += KS)
                        acc = M::mma(frag_t(sC, LN, 16 * ni, k0, lr, lg), yw[k0 / KS], acc);
                    kst[j] = acc;
                    store4(sK + (16 * pj + lr) * LN + 16 * ni + 4 * lg, acc[0], acc[1], acc[2], acc[3]);
                }
            }
        }
        float f_r = 0.f, d_r = 0.f, pre_r = 0.f, cend_r = 0.f;   // wave 0: this block's scalars
        if (w == 0) {
            f_r = sF[lane];
            d_r = sDel[lane];
            pre_r = sPre[lane];
            cend_r = sCend;
        }
        block_sync_lds();

        // ---- phase C: dl, ddt and the per-row sums (wave 0); the next block into LDS and its scalars (wave 1)
        if (w == 0) {
            const int rows = (int)min((int64_t)QB, T - t0);
            float u = 0.f, uo = 0.f, dd = 0.f, cz = 0.f, rz = 0.f;
            if (lane < QB) {
#pragma unroll
                for (int pj = 0; pj < PT; ++pj) {
                    u += sUp[pj][lane];
                    uo += sUop[pj][lane];
                    dd += sDDp[pj][lane];
                }
#pragma unroll
                for (int i = 0; i < QT; ++i) {
                    cz += sCz[i][lane];
                    rz += sRz[i][lane];
                }
            }
            float kap = 0.f;
#pragma unroll
            for (int i = 0; i < NW; ++i) kap += sKap[i];
            const bool valid = lane < rows;
            const float f = lane < QB ? f_r : 0.f;
            // dl_t = [sum_{k<t} (c_k - rho_k)] + [sum_{s>=t} qoff_s] + [sum_{r<t} roff_r] + 2^cend <K, H_in>
            const acc_t zv = lane < QB ? (acc_t)cz - (acc_t)rz : (acc_t)0;
            const acc_t qv = valid ? (acc_t)qcur : (acc_t)0;
            const acc_t rv = lane < QB ? (acc_t)f * (acc_t)uo : (acc_t)0;
            const acc_t zi = wave_incl_scan(zv), qi = wave_incl_scan(qv), ri = wave_incl_scan(rv);
            const acc_t qtot = lane_value<63>(qi);
            const acc_t dl = (zi - zv) + (qtot - qi + qv) + (ri - rv) + (acc_t)cend_r * (acc_t)kap;
            if (valid) {
                const float d = d_r;
                const float a = expf(d * Anat);                   // a_t
                const float fD = fdmode == 1 ? 1.f : (fdmode == 2 ? a : 0.f);
                const float fA = fdmode == 2 ? (d * Anat * a - a + 1.f) / (Anat * Anat) : 0.f;
                float gdt = (float)dl * Anat + u * fD;
                if (prm.dt_softplus) gdt *= 1.f / (1.f + expf(-pre_r));
                prm.ddt[(tb + t0 + lane) * H + h] = gdt;
                sum_dA += dl * (acc_t)d + (acc_t)(u * fA);
                sum_bias += (acc_t)gdt;
                sum_D += (acc_t)dd;
            }
        }
        if (blk > 0) {
            stg.store(sX, sDY, sB, sC, tid);
            if (w == 1) scalars(blk - 1);
            qcur = nxt;                       // (wave 0: nxt is qoff)
        }
        block_sync_lds();
    }

    // dinit = a_0 G_0 = the K that leaves the first block (with no token: dfinal for a
    // row, whose final state is its initial state; 0 for a sequence that does not occur)
    if (prm.seqtab && nblk == 0) {
#pragma unroll
        for (int j = 0; j < K::T_NP; ++j) kst[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (item_dinit) {
#pragma unroll
        for (int j = 0; j < K::T_NP; ++j) {
            const int tile = w + NW * j;
            if (tile < NTL * PT) {
                const int n0 = 16 * (tile / PT) + 4 * lg, p = 16 * (tile % PT) + lr;
                *(float4*)(item_dinit + p * N + n0) = make_float4(kst[j][0], kst[j][1], kst[j][2], kst[j][3]);
            }
        }
    }
    if (w == 0) {
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            sum_dA += __shfl_xor(sum_dA, d);
            sum_bias += __shfl_xor(sum_bias, d);
            sum_D += __shfl_xor(sum_D, d);
        }
        if (lane == 0) {
            prm.part[bh * 3 + 0] = (float)sum_dA;
            prm.part[bh * 3 + 1] = (float)sum_bias;
            prm.part[bh * 3 + 2] = (float)sum_D;
        }
    }
}

// ------------------------------------------------------------ reverse local pass
// For rows split into segments: the gradient that segment j > 0 alone sends to
// the state before it (zero gradient entering its end), K <- 2^cend K +
// dY^T diag(2^cum) C block by block from its last block, and the decay across
// the segment.  The reverse counterpart of the forward's local pass; a combine
// step then chains the segments from the row's end.  One workgroup per (row,
// head, segment j > 0); results at (row, head, j - 1).
template <typename TI, int P, int N, int QB>
__global__ __launch_bounds__((64 * BwdWaves<TI, P, N, QB>::KLOC)) void ssd_bwd_klocal_kernel(BwdParams prm, float* kloc, float* kcarry) {
    using K = BwdCfg<TI, P, N, QB, BwdWaves<TI, P, N, QB>::KLOC>;
    using M = Mfma<TI>;
    typedef typename CumType<TI>::type cum_t;
    constexpr int NW = K::NW, NT = K::NT, LP = K::LP, LN = K::LN, PT = K::PT, NTL = K::NTL, SZ = K::SZ;
    constexpr int KS = M::KSTEP;
    __shared__ __attribute__((aligned(16))) TI sDY[QB * LP];
    __shared__ __attribute__((aligned(16))) TI sC[QB * LN];
    __shared__ __attribute__((aligned(16))) float sDin[64];
    __shared__ float sCend;

    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t H = prm.H, G = prm.G, S1 = prm.nseg - 1;
    const int64_t item = blockIdx.x;                   // (row * H + head) * S1 + j - 1
    const int64_t bh = item / S1, j = item % S1 + 1;
    const int64_t b = bh / H, h = bh % H, g = h / (H / G);
    const int64_t s0 = min(j * prm.seg_tokens, prm.T), T = min(prm.seg_tokens, prm.T - s0), tb = b * prm.T + s0;
    const int nblk = (int)((T + QB - 1) / QB);
    const int ys = (int)(H * P * 4), bs = (int)(G * N * SZ);
    const char* yrow = (const char*)prm.dy + (tb * H + h) * P * 4;
    const char* crow = (const char*)prm.C + (tb * G + g) * N * SZ;
    cum_t A2;
    if constexpr (sizeof(cum_t) == 8) A2 = -exp((double)prm.A_log[h]) * 1.4426950408889634;
    else A2 = -expf(prm.A_log[h]) * 1.4426950408889634f;
    const float dtb = prm.dt_bias ? prm.dt_bias[h] : 0.f;

    f32x4 kst[K::T_NP];
#pragma unroll
    for (int q = 0; q < K::T_NP; ++q) kst[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    cum_t total = 0;                                   // wave 0: log2 decay across the segment
    // dy and C of a block are requested one block ahead (registers), then written to
    // LDS (dy converted to the input type) while the next block's are in flight
    constexpr int YC = P / 4, CC = N * SZ / 16, VE = 16 / SZ;
    constexpr int YU = QB * YC, CU = QB * CC, YPT = (YU + NT - 1) / NT, CPT = (CU + NT - 1) / NT;
    uint4 yv[YPT], cv[CPT];
    float dtn = 0.f;                                   // wave 0: the block's dt (lane = token)
    auto issue = [&](int blk) {
        const int64_t t0 = (int64_t)blk * QB;
        const rsrc_t ry = make_rsrc(yrow + t0 * ys, (T - t0) * ys);
        const rsrc_t rc = make_rsrc(crow + t0 * bs, (T - t0) * bs);
#pragma unroll
        for (int q = 0; q < YPT; ++q) {
            const int v = tid + q * NT;
            if (YU % NT == 0 || v < YU) yv[q] = buf_load16(ry, (v / YC) * ys + (v % YC) * 16);
        }
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int v = tid + q * NT;
            if (CU % NT == 0 || v < CU) cv[q] = buf_load16(rc, (v / CC) * bs + (v % CC) * 16);
        }
        if (w == 0) dtn = buf_load_f32(make_rsrc(prm.dt + (b * H + h) * prm.T + s0 + t0, (T - t0) * 4), lane * 4);
    };
    auto stage = [&](int blk) {
#pragma unroll
        for (int q = 0; q < YPT; ++q) {
            const int v = tid + q * NT;
            if (YU % NT == 0 || v < YU) {
                const float4 f = __builtin_bit_cast(float4, yv[q]);
                store4(sDY + (v / YC) * LP + (v % YC) * 4, f.x, f.y, f.z, f.w);
            }
        }
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int v = tid + q * NT;
            if (CU % NT == 0 || v < CU) *(uint4*)(sC + (v / CC) * LN + (v % CC) * VE) = cv[q];
        }
        if (w == 0) {
            const int rows = (int)min((int64_t)QB, T - (int64_t)blk * QB);
            const float d = lane < rows ? step_size(dtn + dtb, prm.dt_softplus) : 0.f;
            const cum_t cum = wave_incl_scan((cum_t)d * A2);
            const cum_t cend = lane_value<QB - 1>(cum);
            if (lane < QB) sDin[lane] = fast_exp2((float)cum);
            if (lane == 0) sCend = fast_exp2((float)cend);
            total += cend;
        }
    };
    if (nblk > 0) issue(nblk - 1);
    for (int blk = nblk - 1; blk >= 0; --blk) {
        stage(blk);
        if (blk > 0) issue(blk - 1);
        block_sync_lds();
        const float dec = sCend;
        // every state tile of this wave has channel tile w mod PT: its weighted dY
        // operands are formed once for all of them
        static_assert(NW % PT == 0, "a wave's state tiles share one channel tile");
        decltype(frag_t_w(sDY, LP, 0, 0, lr, lg, sDin)) yw[QB / KS];
#pragma unroll
        for (int k0 = 0; k0 < QB; k0 += KS) yw[k0 / KS] = frag_t_w(sDY, LP, 16 * (w % PT), k0, lr, lg, sDin);
#pragma unroll
        for (int q = 0; q < K::T_NP; ++q) {
            const int tile = w + NW * q;
            if (tile < NTL * PT) {
                const int ni = tile / PT;
                f32x4 acc = kst[q] * dec;
#pragma unroll
                for (int k0 = 0; k0 < QB; k0 += KS) acc = M::mma(frag_t(sC, LN, 16 * ni, k0, lr, lg), yw[k0 / KS], acc);
                kst[q] = acc;
            }
        }
        block_sync_lds();
    }
    float* dst = kloc + item * (int64_t)(P * N);
#pragma unroll
    for (int q = 0; q < K::T_NP; ++q) {
        const int tile = w + NW * q;
        if (tile < NTL * PT) {
            const int n0 = 16 * (tile / PT) + 4 * lg, p = 16 * (tile % PT) + lr;
            *(float4*)(dst + p * N + n0) = make_float4(kst[q][0], kst[q][1], kst[q][2], kst[q][3]);
        }
    }
    if (w == 0 && lane == 0) kcarry[item] = fast_exp2((float)total);
}

}  // namespace ssd
