// Attention backward pass, bf16 in / bf16 out, fp32 accumulation, head size
// 64, for gfx950.  For O = softmax(S) V, S = Q K^T * scale + M, and the
// upstream gradient dO, the gradients taken through the forward's steps in
// reverse order are
//
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O),
//   dQ = scale * dS K,  dK = scale * dS^T Q
//
// (the forward's definition: devpress.csdn.net "【深度学习】Transformer",
// section 2.1, equation (2.4); training back-propagates the losses of all
// positions at once: hex4c59.cc "读懂 Attention Is All You Need", sections
// "训练能并行，不意味着一次生成整句话" and "参数是怎样学出来的？").  P is not
// stored by the forward: it is recomputed from S and the row log-sum-exp
// the forward saved, P = exp(S - lse), one exponential per entry, no row
// reductions.  The per-row constants enter the score products as their
// initial accumulators (fp32, exact): the raw-score product starts at
// -lse/scale, so it yields (S - lse)/scale and P = exp2(acc * scale log2 e);
// the dP product starts at -D, so it yields dP - D and dS = P * acc.  The dQ
// kernel writes both row constants, -lse/scale and -D, to the workspace.
//
// Two kernels, deterministic (no atomics):
//   attn_bwd_dq_kernel    workgroup = 128 queries of one (batch, head), wave
//                         = 32 queries; streams the K/V tiles like the
//                         forward; lane = query (S^T, dP^T layouts), so P
//                         and dS need the lane's own lse and D only.  Writes
//                         dQ and D (the dK/dV kernel reads D).
//   attn_bwd_dkdv_kernel  workgroup = 128 keys, wave = 32 keys; streams the
//                         Q/dO tiles (64 queries, with their lse and D);
//                         lane = key (S, dP layouts).
// Per 32 x 64 block a wave runs 32 MFMA 32x32x16 (two score-shaped
// products, two accumulations).  The accumulation operands come from
// transposing LDS reads (ds_read_b64_tr_b16) in the key (or query) order of
// the score product's output rows, the same scheme as the forward's P V.
#include "wave_attention.h"

namespace mha {
namespace {

using namespace dev;

constexpr int NW = 4;                   // waves per workgroup
constexpr int BT = 64;                  // rows per streamed tile (keys or queries)
constexpr int CHW = BT * D * 2 / 1024 / NW;  // 1 KB copies per wave and tile (2)
constexpr float kLog2e = 1.4426950408889634f;

// Offsets (elements) of this lane's transposing reads: within each 16-lane
// group, lane s addresses row (s / 4) (+4 for lane group g = 1) and columns
// 4 (s % 4) .. +3 of its 16-wide column block; db selects columns 0..31 or
// 32..63 (v_off layout).
__device__ __forceinline__ void tr_offsets(int lane, int vx[2]) {
  const int g = lane >> 5;
  const int tr_row = ((lane & 15) >> 2) + 4 * g;
  const int tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const int c = 32 * db + tr_c;
    vx[db] = v_off(tr_row, c >> 3) + (c & 7);
  }
}

// acc{0,1} (columns 0..31, 32..63 of the product's rows) += T^T . W for the
// 32 rows of half h of a [64][64] v_off-layout tile T (rows 32h .. 32h+31 in
// two 16-row steps) and W = (wa, wb), the matching rows' values in the
// order of a score product's output rows.
__device__ __forceinline__ void acc_half(const __bf16* t, const int vx[2], int h, const bf16x8& wa,
                                         const bf16x8& wb, f32x16& acc0, f32x16& acc1) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int kk = 2 * h + j;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const i16x4 lo = tr_read(&t[vx[db] + 16 * kk * D]);
      const i16x4 hi = tr_read(&t[vx[db] + (16 * kk + 8) * D]);
      const bf16x8 ta = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      const bf16x8& w = j == 0 ? wa : wb;
      if (db == 0) acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta, w, acc0, 0, 0, 0);
      else acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta, w, acc1, 0, 0, 0);
    }
  }
}

// A row (64 bf16) of this lane's own query or key as the score product's
// per-lane operand: f[s] = row[16 s + 8 g .. +7].
__device__ __forceinline__ void load_row_operand(const __bf16* row, int g, bf16x8 f[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) f[s] = ((const bf16x8*)row)[2 * s + g];
}

// 32 x 32 score-shaped product over d = 64 added to the accumulator init:
// rows from an LDS tile in the k_off layout (row offsets rx), columns from
// the lane's own operand f.
__device__ __forceinline__ f32x16 score32(const __bf16* t, const int rx[4], int row0, const bf16x8 f[4],
                                          f32x16 s) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const bf16x8 a = *(const bf16x8*)&t[rx[kk] + row0 * D];
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, f[kk], s, 0, 0, 0);
  }
  return s;
}

// Source column chunk that lands in stored chunk (q & 7) of row (q >> 3)
// under the k_off (row reads) and v_off (transposing reads) swizzles.
__device__ __forceinline__ void swz(int q, int& row, int& kc, int& vc) {
  row = q >> 3;
  kc = ((q & 7) ^ ((row >> 1) & 7)) * 8;
  vc = ((q & 7) ^ (((row >> 1) & 1) << 2)) * 8;
}

// ---------------------------------------------------------------------- dQ

// Three waves per SIMD (48 KB of LDS: three workgroups per compute unit):
// at most 168 registers per lane, accumulators included.
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(3, 3)))
void attn_bwd_dq_kernel(const BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) __bf16 Ks[2][BT * D];  // K, k_off (score rows)
  __shared__ __attribute__((aligned(1024))) __bf16 Kt[2][BT * D];  // K, v_off (dS K)
  __shared__ __attribute__((aligned(1024))) __bf16 Vs[2][BT * D];  // V, k_off (dP rows)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31;
  const int g = lane >> 5;
  const int bh = blockIdx.x;
  const int b = __builtin_amdgcn_readfirstlane(bh / a.h);
  const int qt = (int)gridDim.y - 1 - (int)blockIdx.y;  // heaviest causal tiles first
  const int q0 = qt * NW * 32;
  const int64_t qbase = (int64_t)bh * a.n_q * D;
  const int64_t kbase = (int64_t)bh * a.n_k * D;
  const char* Kp = wave_uniform((const char*)((const __bf16*)a.K + kbase));
  const char* Vp = wave_uniform((const char*)((const __bf16*)a.V + kbase));

  int L = a.n_k;
  if (a.padded) L = min(L, a.key_len[b]);
  const int qw0 = q0 + 32 * wave;
  const int my_q = qw0 + col;
  const int qc = min(my_q, a.n_q - 1);
  const int lim = a.causal ? min(L, my_q + 1) : L;
  const int lim_min = __builtin_amdgcn_readfirstlane(a.causal ? min(L, qw0 + 1) : L);
  const int wg_last = min(q0 + NW * 32, a.n_q) - 1;
  const int wg_keys = a.causal ? min(L, wg_last + 1) : L;
  const int wv_last = min(qw0 + 32, a.n_q) - 1;
  const int wv_keys =
      __builtin_amdgcn_readfirstlane(wv_last < qw0 ? 0 : (a.causal ? min(L, wv_last + 1) : L));
  const int ntiles = __builtin_amdgcn_readfirstlane((wg_keys + BT - 1) / BT);

  // The lane's query: Q and dO rows as operands, D = dO . O, log2-domain lse.
  bf16x8 qf[4], dof[4];
  const __bf16* qrow = (const __bf16*)a.Q + qbase + (int64_t)qc * D;
  const __bf16* dorow = (const __bf16*)a.dO + qbase + (int64_t)qc * D;
  load_row_operand(qrow, g, qf);
  load_row_operand(dorow, g, dof);
  float dpart = 0.f;
  {
    const __bf16* orow = (const __bf16*)a.O + b * a.o_sb + (int64_t)(bh - b * a.h) * a.o_sh + (int64_t)qc * a.o_sr;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 o8 = ((const bf16x8*)orow)[4 * g + c];
      const bf16x8 d8 = ((const bf16x8*)dorow)[4 * g + c];
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart = fmaf((float)d8[e], (float)o8[e], dpart);
    }
  }
  const float Dq = sum_halves(dpart);
  const float ls = -a.lse[(int64_t)bh * a.n_q + qc] / a.scale;  // -lse / scale
  if (g == 0 && my_q < a.n_q) {
    a.Dw[(int64_t)bh * a.n_q + my_q] = -Dq;
    a.Lw[(int64_t)bh * a.n_q + my_q] = ls;
  }
  const float c2 = a.scale * kLog2e;
  f32x16 s_init, dp_init;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    s_init[i] = ls;
    dp_init[i] = -Dq;
  }

  int kx[4], vx[2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) kx[kk] = k_off(col, 2 * kk + g);
  tr_offsets(lane, vx);

  // Copies: wave w fills 1 KB blocks 2w, 2w+1 of each tile (rows 8 blk .. +7).
  const unsigned ks_lds = lds_addr(&Ks[0][0]), kt_lds = lds_addr(&Kt[0][0]), vs_lds = lds_addr(&Vs[0][0]);
  auto issue = [&](int tile, int buf) {
    const int k0 = tile * BT;
    // 64-bit base of the tile's first row; per-lane offsets stay small
    const char* kb = wave_uniform(Kp + (int64_t)k0 * D * 2);
    const char* vb = wave_uniform(Vp + (int64_t)k0 * D * 2);
#pragma unroll
    for (int r = 0; r < CHW; ++r) {
      int row, kc, vc;
      swz((wave * CHW + r) * 64 + lane, row, kc, vc);
      const int rr = min(row, a.n_k - 1 - k0);  // rows past n_k repeat the last (masked)
      const unsigned dst = (unsigned)(buf * BT * D * 2 + (wave * CHW + r) * 1024);
      dma16_s(kb, (unsigned)(rr * D + kc) * 2u, ks_lds + dst);
      dma16_s(kb, (unsigned)(rr * D + vc) * 2u, kt_lds + dst);
      dma16_s(vb, (unsigned)(rr * D + kc) * 2u, vs_lds + dst);
    }
  };

  f32x16 dq0 = {}, dq1 = {};
  if (ntiles > 0) issue(0, 0);
  for (int t0 = 0; t0 < ntiles; t0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = t0 + u;
      if (t < ntiles) {
        wait_vmcnt<0>();
        __syncthreads();
        if (t + 1 < ntiles) issue(t + 1, u ^ 1);
        const int k0 = t * BT;
        if (k0 < wv_keys) {
#pragma unroll
          for (int hk = 0; hk < 2; ++hk) {
            const f32x16 s = score32(Ks[u], kx, 32 * hk, qf, s_init);     // (S^T - lse) / scale
            const f32x16 dp = score32(Vs[u], kx, 32 * hk, dof, dp_init);  // dP^T - D
            bf16x8 wa, wb;
            f32x8 w0, w1;
            float p[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) p[i] = fast_exp2(s[i] * c2);
            if (k0 + 32 * hk + 32 > lim_min) {  // wave-uniform: a tile on the mask's edge
#pragma unroll
              for (int i = 0; i < 16; ++i)
                if (k0 + 32 * hk + 8 * (i >> 2) + 4 * g + (i & 3) >= lim) p[i] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float ds = p[i] * dp[i];
              if (i < 8) w0[i] = ds;
              else w1[i - 8] = ds;
            }
            wa = __builtin_convertvector(w0, bf16x8);
            wb = __builtin_convertvector(w1, bf16x8);
            acc_half(Kt[u], vx, hk, wa, wb, dq0, dq1);    // dQ^T += K^T dS^T
          }
        }
      }
    }
  }
  wait_vmcnt<0>();
  store_row_bf16((__bf16*)a.dQ + b * a.dq_sb + (int64_t)(bh - b * a.h) * a.dq_sh +
                     (int64_t)min(my_q, a.n_q - 1) * a.dq_sr,
                 g, dq0, dq1, a.scale, my_q < a.n_q);
}

// ---------------------------------------------------------------- dK and dV

// Two waves per SIMD (65 KB of LDS: two workgroups per compute unit): at
// most 256 registers per lane, accumulators included.
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv_kernel(const BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) __bf16 Qs[2][BT * D];   // Q, k_off (score rows)
  __shared__ __attribute__((aligned(1024))) __bf16 Qt[2][BT * D];   // Q, v_off (dS^T Q)
  __shared__ __attribute__((aligned(1024))) __bf16 Os[2][BT * D];   // dO, k_off (dP rows)
  __shared__ __attribute__((aligned(1024))) __bf16 Ot[2][BT * D];   // dO, v_off (P^T dO)
  __shared__ __attribute__((aligned(256))) float Ls[2][BT];          // -lse / scale
  __shared__ __attribute__((aligned(256))) float Ds[2][BT];          // -D

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31;
  const int g = lane >> 5;
  const int bh = blockIdx.x;
  const int b = __builtin_amdgcn_readfirstlane(bh / a.h);
  const int k0 = (int)blockIdx.y * NW * 32;
  const int64_t qbase = (int64_t)bh * a.n_q * D;
  const int64_t kbase = (int64_t)bh * a.n_k * D;
  const char* Qp = wave_uniform((const char*)((const __bf16*)a.Q + qbase));
  const char* dOp = wave_uniform((const char*)((const __bf16*)a.dO + qbase));

  int L = a.n_k;
  if (a.padded) L = min(L, a.key_len[b]);
  const int kw0 = k0 + 32 * wave;
  const int my_k = kw0 + col;
  const int kc_ = min(my_k, a.n_k - 1);
  // Query tiles: causal -> from the tile holding the workgroup's first key.
  const int t_first = a.causal ? k0 / BT : 0;
  const int ntiles = (a.n_q + BT - 1) / BT;
  const bool wave_live = kw0 < L;  // some key of this wave is visible to someone

  bf16x8 kf[4], vf[4];
  load_row_operand((const __bf16*)a.K + kbase + (int64_t)kc_ * D, g, kf);
  load_row_operand((const __bf16*)a.V + kbase + (int64_t)kc_ * D, g, vf);
  const float c2 = a.scale * kLog2e;

  int qx[4], vx[2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qx[kk] = k_off(col, 2 * kk + g);
  tr_offsets(lane, vx);

  const unsigned qs_lds = lds_addr(&Qs[0][0]), qt_lds = lds_addr(&Qt[0][0]);
  const unsigned os_lds = lds_addr(&Os[0][0]), ot_lds = lds_addr(&Ot[0][0]);
  const unsigned ls_lds = lds_addr(&Ls[0][0]), ds_lds = lds_addr(&Ds[0][0]);
  const char* Lp = wave_uniform((const char*)(a.Lw + (int64_t)bh * a.n_q));
  const char* Dp = wave_uniform((const char*)(a.Dw + (int64_t)bh * a.n_q));
  auto issue = [&](int tile, int buf) {
    const int q0 = tile * BT;
    // 64-bit bases of the tile's first row; per-lane offsets stay small
    const char* qb = wave_uniform(Qp + (int64_t)q0 * D * 2);
    const char* ob = wave_uniform(dOp + (int64_t)q0 * D * 2);
#pragma unroll
    for (int r = 0; r < CHW; ++r) {
      int row, kc, vc;
      swz((wave * CHW + r) * 64 + lane, row, kc, vc);
      const int rr = min(row, a.n_q - 1 - q0);  // rows past n_q repeat the last (masked)
      const unsigned dst = (unsigned)(buf * BT * D * 2 + (wave * CHW + r) * 1024);
      dma16_s(qb, (unsigned)(rr * D + kc) * 2u, qs_lds + dst);
      dma16_s(qb, (unsigned)(rr * D + vc) * 2u, qt_lds + dst);
      dma16_s(ob, (unsigned)(rr * D + kc) * 2u, os_lds + dst);
      dma16_s(ob, (unsigned)(rr * D + vc) * 2u, ot_lds + dst);
    }
    // -lse/scale and -D of the tile's 64 queries: one 4-byte copy per lane
    const unsigned qo = (unsigned)min(lane, a.n_q - 1 - q0) * 4u;
    if (wave == 0) dma4_s(Lp + (int64_t)q0 * 4, qo, ls_lds + (unsigned)(buf * BT * 4));
    if (wave == 1) dma4_s(Dp + (int64_t)q0 * 4, qo, ds_lds + (unsigned)(buf * BT * 4));
  };

  f32x16 dk0 = {}, dk1 = {}, dv0 = {}, dv1 = {};
  if (t_first < ntiles) issue(t_first, 0);
  for (int t0 = t_first; t0 < ntiles; t0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = t0 + u;
      if (t < ntiles) {
        wait_vmcnt<0>();
        __syncthreads();
        if (t + 1 < ntiles) issue(t + 1, u ^ 1);
        const int q0 = t * BT;
        // the tile's last query sees some key of this wave (causal), or no causal mask
        if (wave_live && (!a.causal || q0 + BT - 1 >= kw0)) {
          // every (query, key) pair of the tile and the wave visible: no per-element test
          const bool full = kw0 + 32 <= L && q0 + BT <= a.n_q && (!a.causal || q0 >= kw0 + 31);
#pragma unroll
          for (int hq = 0; hq < 2; ++hq) {
            // element 4 i4 + r of a lane is query row 32 hq + 8 i4 + 4 g + r of the tile
            f32x16 s_init, dp_init;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const int qr = 32 * hq + 8 * i4 + 4 * g;
              const f32x4 l4 = *(const f32x4*)&Ls[u][qr];
              const f32x4 d4 = *(const f32x4*)&Ds[u][qr];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                s_init[4 * i4 + r] = l4[r];
                dp_init[4 * i4 + r] = d4[r];
              }
            }
            const f32x16 s = score32(Qs[u], qx, 32 * hq, kf, s_init);    // (S - lse) / scale
            const f32x16 dp = score32(Os[u], qx, 32 * hq, vf, dp_init);  // dP - D
            float p[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) p[i] = fast_exp2(s[i] * c2);
            if (!full) {  // wave-uniform: a tile on the mask's edge
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int q = q0 + 32 * hq + 8 * (i >> 2) + 4 * g + (i & 3);
                if (!(my_k < L && q < a.n_q && (!a.causal || my_k <= q))) p[i] = 0.f;
              }
            }
            f32x8 p0, p1, w0, w1;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              p0[i] = p[i];
              p1[i] = p[8 + i];
              w0[i] = p[i] * dp[i];
              w1[i] = p[8 + i] * dp[8 + i];
            }
            const bf16x8 pa = __builtin_convertvector(p0, bf16x8), pb = __builtin_convertvector(p1, bf16x8);
            const bf16x8 wa = __builtin_convertvector(w0, bf16x8), wb = __builtin_convertvector(w1, bf16x8);
            acc_half(Ot[u], vx, hq, pa, pb, dv0, dv1);   // dV^T += dO^T P
            acc_half(Qt[u], vx, hq, wa, wb, dk0, dk1);   // dK^T += Q^T dS
          }
        }
      }
    }
  }
  wait_vmcnt<0>();
  const int64_t hh = bh - b * a.h;
  const int64_t kr = min(my_k, a.n_k - 1);
  store_row_bf16((__bf16*)a.dK + b * a.dk_sb + hh * a.dk_sh + kr * a.dk_sr, g, dk0, dk1, a.scale, my_k < a.n_k);
  store_row_bf16((__bf16*)a.dV + b * a.dv_sb + hh * a.dv_sh + kr * a.dv_sr, g, dv0, dv1, 1.0f, my_k < a.n_k);
}

}  // namespace

hipError_t launch_attn_bwd_dq(const BwdArgs& a, hipStream_t s, LaunchEvents ev) {
  void* args[] = {(void*)&a};
  dim3 grid(a.B * a.h, (a.n_q + NW * 32 - 1) / (NW * 32));
  return launch_kernel((const void*)attn_bwd_dq_kernel, grid, dim3(NW * 64), args, 0, s,
                            ev.start, ev.stop, 0);
}

hipError_t launch_attn_bwd_dkdv(const BwdArgs& a, hipStream_t s, LaunchEvents ev) {
  void* args[] = {(void*)&a};
  dim3 grid(a.B * a.h, (a.n_k + NW * 32 - 1) / (NW * 32));
  return launch_kernel((const void*)attn_bwd_dkdv_kernel, grid, dim3(NW * 64), args, 0, s,
                            ev.start, ev.stop, 0);
}

}  // namespace mha
