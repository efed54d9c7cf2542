// kda_intra.hip -- intra-chunk stage of the KDA chunked forward for gfx950.
//
// One workgroup (4 waves) per (chunk of 64 tokens, value head).  From q, k, g,
// beta it computes, following the kernel-fun fwd_state module docstring (the
// operands the state scan consumes) and the FlashKDA walkthrough (INV, Mqk):
//   Gam      = inclusive cumsum of g over the chunk (per key dimension)
//   qg       = scale * q * exp(Gam)
//   kg       = k * exp(Gam_last - Gam)
//   Aqk[i,j] = scale * sum_d q_id k_jd exp(Gam_id - Gam_jd),   j <= i
//   Akk[i,j] = beta_i * sum_d k_id k_jd exp(Gam_id - Gam_jd),  j <  i
//   Tm       = (I + Akk)^-1 ;  TmB = Tm diag(beta) ;  w = TmB (k * exp(Gam))
// and writes them as one workspace record in the inter kernel's fragment order
// (kda_device.hpp).
//
// Gate factoring.  exp(Gam_i - Gam_j) inside the d-sum cannot be pulled out, so
// each 16-row block I gets a per-dimension reference mu_I (its cumsum midpoint)
// and the factors X_i = exp(Gam_i - mu_I), Y_j = exp(mu_I - Gam_j):
//   same block:   exp(Gam_i - Gam_j) = X_i Y_j
//   block J < I:  exp(Gam_i - Gam_j) = X_i * exp(mu_I - mu_J) * Y_j
// so Aqk/Akk run on bf16 MFMA with two exponentials per element.  Each factor is
// bounded by exp(8 |g|) (half a block of decay), which stays finite for per-token
// gates g >= -11 (natural log).  The Gam-referenced outputs are rebuilt from the
// same factors: exp(Gam_i) = X_i exp(mu_I), exp(Gam_last - Gam_i) = Y_i exp(Gam_last - mu_I).
//
// Wave I owns rows 16I..16I+15 through the gate and Aqk/Akk phases; lane
// l = 16g + r holds row 16I + r and key dims 32s + 8g .. +7 (s = 0..K/32-1),
// which is at once the MFMA A/B fragment layout and the qg record layout.

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

template <int K>
struct IntraSmem {
  static constexpr int S = K / 32;
  static constexpr int TS = 72;                         // transposed-tile row stride (bf16)
  static constexpr int TOT = 0;                         // float [4][K] block gate totals
  static constexpr int TAB = TOT + 4 * K * 4;           // float [14][K] E, F, c tables
  static constexpr int BETA = TAB + 14 * K * 4;         // float [64]
  static constexpr int KY = BETA + 256;                 // float [4][S][64][8] k*Y fragments
  static constexpr int KDT = KY + 4 * S * 64 * 8 * 4;   // bf16 [K][TS] (k*exp(Gam))^T
  static constexpr int KGT = KDT + K * TS * 2;          // bf16 [K][TS] kg^T
  static constexpr int END0 = KGT + K * TS * 2;
  static constexpr int AS = 68;                         // Akk / Tm row stride (fp32)
  static constexpr int AKK_BYTES = 64 * AS * 4;
  static constexpr int AKK = (K * TS * 2 >= AKK_BYTES) ? KGT : END0;   // reuses kg^T when it fits
  static constexpr int STG_S = K + 8;                   // staging row stride (bf16)
  static constexpr int STG = KY;                        // bf16 [64][STG_S], reuses k*Y
  static_assert(64 * STG_S * 2 <= 4 * S * 64 * 8 * 4, "staging fits in the k*Y area");
  static_assert(64 * 72 * 2 <= 4 * S * 64 * 8 * 4, "Aqk staging fits in the k*Y area");
  static constexpr int BYTES = (AKK == KGT) ? END0 : END0 + AKK_BYTES;
};

// Row of the transposed [K][64] tiles: 8-token groups are XOR-swizzled by
// (d >> 3) & 3 on bits 4-5 so that the column writes of a wave spread over the
// LDS banks while every 8-token group stays contiguous (16-byte reads).
__device__ __forceinline__ int tcol(int t, int d) { return t ^ (((d >> 3) & 3) << 4); }

struct ChunkLoc {
  int b;
  int64_t row0;  // first row of the chunk within batch row b
  int L;         // valid rows (1..64)
};

// Chunk gc -> (batch row, first row, valid rows).  Returns false when gc is past
// the last chunk (varlen capacity padding) or the chunk table was rejected.
__device__ __forceinline__ bool locate_chunk(const Params& p, int64_t gc, ChunkLoc& c) {
  if (p.cu == nullptr) {
    int n = (int)(gc / p.NT);
    if (n >= p.B) return false;
    c.b = n;
    c.row0 = (gc - (int64_t)n * p.NT) * BT;
    c.L = (int)min<int64_t>(BT, p.T - c.row0);
    return c.L > 0;
  }
  const int32_t* tb = p.table;
  if (tb[p.N + 1] != 0 || gc >= tb[p.N]) return false;
  int lo = 0, hi = p.N - 1;  // last n with tb[n] <= gc
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (tb[mid] <= gc) lo = mid; else hi = mid - 1;
  }
  c.b = 0;
  c.row0 = p.cu[lo] + (gc - tb[lo]) * BT;
  c.L = (int)min<int64_t>(BT, p.cu[lo + 1] - c.row0);
  return c.L > 0;
}

// ----------------------------------------------------------- chunk table
// One workgroup: chunk_base[n] = sum_{m<n} ceil(len_m / 64) (the tile_base of the
// FlashKDA walkthrough's sequence-information section), chunk_base[N] = total,
// and an error flag at [N+1] if cu_seqlens is not 0 = cu[0] <= ... <= cu[N] = T.
__global__ __launch_bounds__(256) void chunk_table_kernel(Params p) {
  __shared__ int32_t scan[256];
  __shared__ int32_t bad_any;
  const int tid = threadIdx.x;
  if (tid == 0) bad_any = (p.cu[0] != 0 || p.cu[p.N] != p.T) ? 1 : 0;
  __syncthreads();
  int32_t running = 0;
  for (int base = 0; base < p.N; base += 256) {
    const int n = base + tid;
    int32_t cnt = 0;
    if (n < p.N) {
      const int64_t a = p.cu[n], e = p.cu[n + 1];
      if (a < 0 || e < a || e > p.T) atomicOr(&bad_any, 1);
      else cnt = (int32_t)((e - a + BT - 1) / BT);
    }
    scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      int32_t add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    if (n < p.N) p.table[n] = running + scan[tid] - cnt;
    running += scan[255];
    __syncthreads();
  }
  if (tid == 0) {
    p.table[p.N] = running;
    p.table[p.N + 1] = (bad_any || running > p.max_chunks) ? 1 : 0;
  }
}

// ------------------------------------------------------------ intra kernel
template <int K>
__global__ __launch_bounds__(NTHREADS, 2) void intra_kernel(Params p, int n_items) {
  using SM = IntraSmem<K>;
  using R = Rec<K>;
  constexpr int S = SM::S;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SM::BYTES];
  float* sTot = reinterpret_cast<float*>(smem + SM::TOT);
  float* sTab = reinterpret_cast<float*>(smem + SM::TAB);
  float* sBeta = reinterpret_cast<float*>(smem + SM::BETA);
  float* sKY = reinterpret_cast<float*>(smem + SM::KY);
  uint16_t* sKdT = reinterpret_cast<uint16_t*>(smem + SM::KDT);
  uint16_t* sKgT = reinterpret_cast<uint16_t*>(smem + SM::KGT);
  float* sAkk = reinterpret_cast<float*>(smem + SM::AKK);
  uint16_t* sStg = reinterpret_cast<uint16_t*>(smem + SM::STG);

  const int item = xcd_remap(blockIdx.x, gridDim.x);
  if (item >= n_items) return;
  const int hv = item % p.HV;
  const int64_t gc = item / p.HV;
  ChunkLoc cl;
  if (!locate_chunk(p, gc, cl)) return;
  const int hq = hv / (p.HV / p.HQK);

  const int tid = threadIdx.x;
  const int wv = tid >> 6;        // row block I
  const int ln = tid & 63;
  const int r = ln & 15, grp = ln >> 4;
  const int i = 16 * wv + r;      // this lane's row in the chunk
  const bool valid = i < cl.L;
  const int64_t tok = (int64_t)cl.b * p.T + cl.row0 + i;
  uint8_t* rec = p.recs + (gc * p.HV + hv) * (int64_t)R::BYTES;

  // ---- phase 1: loads, gate cumsum, factors -----------------------------------
  float qf[S][8], kf[S][8], gl[S][8];
  {
    const uint16_t* qrow = p.q + (tok * p.HQK + hq) * K;
    const uint16_t* krow = p.k + (tok * p.HQK + hq) * K;
    const uint16_t* grow = p.g + (tok * p.HV + hv) * K;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int d0 = 32 * s + 8 * grp;
      uint4 uq = make_uint4(0, 0, 0, 0), uk = uq, ug = uq;
      if (valid) {
        uq = *reinterpret_cast<const uint4*>(qrow + d0);
        uk = *reinterpret_cast<const uint4*>(krow + d0);
        ug = *reinterpret_cast<const uint4*>(grow + d0);
      }
      unpack8(uq, qf[s]);
      unpack8(uk, kf[s]);
      unpack8(ug, gl[s]);
    }
    const float bt = valid ? bf2f(p.beta[tok * p.HV + hv]) : 0.f;
    if (grp == 0) sBeta[i] = bt;
  }
  // in-block inclusive cumsum over the 16 rows (lanes r = 0..15 of a DPP row)
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) gl[s][e] = row_inclusive_scan(gl[s][e]);
  if (r == 15) {
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) sTot[wv * K + 32 * s + 8 * grp + e] = gl[s][e];
  }
  __syncthreads();  // B1: block totals

  // tables, per key dim d (natural-log sums, exp2 of log2e-scaled arguments):
  //   rows 0..3  E_I = exp(mu_I)            mu_I = prefix_I + tot_I / 2
  //   rows 4..7  F_I = exp(Gam_last - mu_I)
  //   rows 8..13 c_IJ = exp(mu_I - mu_J), pair (I,J) -> 8 + I(I-1)/2 + J
  for (int idx = tid; idx < 14 * K; idx += NTHREADS) {
    const int row = idx / K, d = idx - row * K;
    const float t0 = sTot[d], t1 = sTot[K + d], t2 = sTot[2 * K + d], t3 = sTot[3 * K + d];
    const float mu[4] = {0.5f * t0, t0 + 0.5f * t1, t0 + t1 + 0.5f * t2, t0 + t1 + t2 + 0.5f * t3};
    const float G = t0 + t1 + t2 + t3;
    float a;
    if (row < 4) a = mu[row];
    else if (row < 8) a = G - mu[row - 4];
    else {
      const int pr = row - 8;
      const int I = pr < 1 ? 1 : (pr < 3 ? 2 : 3);
      const int J = pr - I * (I - 1) / 2;
      a = mu[I] - mu[J];
    }
    sTab[idx] = exp2f(LOG2E * a);
  }
  if (tid < K) {
    const int d = tid;
    const float G = sTot[d] + sTot[K + d] + sTot[2 * K + d] + sTot[3 * K + d];
    reinterpret_cast<float*>(rec + R::ALPHA)[d] = exp2f(LOG2E * G);
  }
  __syncthreads();  // B2: tables

  bf16x8 QX[S], KX[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    float qx[8], kx[8], ky[8], qg[8];
    const int d0 = 32 * s + 8 * grp;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = d0 + e;
      const float half = 0.5f * sTot[wv * K + d];
      const float X = exp2f(LOG2E * (gl[s][e] - half));
      const float Y = exp2f(LOG2E * (half - gl[s][e]));
      const float E = sTab[wv * K + d];
      const float F = sTab[(4 + wv) * K + d];
      qx[e] = qf[s][e] * X;
      kx[e] = kf[s][e] * X;
      ky[e] = kf[s][e] * Y;
      qg[e] = p.scale * qx[e] * E;
      sKdT[d * SM::TS + tcol(i, d)] = f2bf(kx[e] * E);
      sKgT[d * SM::TS + tcol(i, d)] = f2bf(ky[e] * F);
    }
    QX[s] = as_frag(pack8(qx));
    KX[s] = as_frag(pack8(kx));
    float4* dst = reinterpret_cast<float4*>(sKY + ((wv * S + s) * 64 + ln) * 8);
    dst[0] = make_float4(ky[0], ky[1], ky[2], ky[3]);
    dst[1] = make_float4(ky[4], ky[5], ky[6], ky[7]);
    *reinterpret_cast<uint4*>(rec + R::QG + ((wv * S + s) * 64 + ln) * 16) = pack8(qg);
  }
  __syncthreads();  // B3: k*Y, kd^T, kg^T

  // ---- phase 2: kg^T record, Aqk / Akk block row I = wv --------------------------
  for (int f = wv; f < 2 * (K / 16); f += 4) {
    const int md = f >> 1, s2 = f & 1;
    const int d = 16 * md + r;
    const uint4 u = *reinterpret_cast<const uint4*>(sKgT + d * SM::TS + tcol(32 * s2 + 8 * grp, d));
    *reinterpret_cast<uint4*>(rec + R::KGT + (f * 64 + ln) * 16) = u;
  }
  f32x4 aq[4], ak[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    aq[J] = f32x4{0.f, 0.f, 0.f, 0.f};
    ak[J] = aq[J];
    if (J > wv) continue;
    const int pr = 8 + wv * (wv - 1) / 2 + J;   // c_IJ table row (J < I)
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const float4* src = reinterpret_cast<const float4*>(sKY + ((J * S + s) * 64 + ln) * 8);
      const float4 a0 = src[0], a1 = src[1];
      float b[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      if (J < wv) {
        const float4* c = reinterpret_cast<const float4*>(sTab + pr * K + 32 * s + 8 * grp);
        const float4 c0 = c[0], c1 = c[1];
        b[0] *= c0.x; b[1] *= c0.y; b[2] *= c0.z; b[3] *= c0.w;
        b[4] *= c1.x; b[5] *= c1.y; b[6] *= c1.z; b[7] *= c1.w;
      }
      const bf16x8 B = as_frag(pack8(b));
      aq[J] = mfma16x32(QX[s], B, aq[J]);
      ak[J] = mfma16x32(KX[s], B, ak[J]);
    }
  }
  __syncthreads();  // B4: k*Y and kg^T reads done (their space is reused below)

  // Akk -> LDS fp32 (full 64 columns of this block row, zeros right of the block
  // diagonal); Aqk -> staging bf16.  C layout: rows 16I + 4grp + rr, column 16J + r.
#pragma unroll
  for (int J = 0; J < 4; ++J) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = 16 * wv + 4 * grp + rr, col = 16 * J + r;
      float vk = 0.f, vq = 0.f;
      if (J < wv || (J == wv && col < row)) vk = sBeta[row] * ak[J][rr];
      if (J < wv || (J == wv && col <= row)) vq = p.scale * aq[J][rr];
      sAkk[row * SM::AS + col] = vk;
      sStg[row * 72 + col] = f2bf(vq);
    }
  }
  __syncthreads();  // B5

  // Aqk record fragments (this wave's row block)
  for (int s2 = 0; s2 < tri_steps(wv); ++s2) {
    const uint4 u = *reinterpret_cast<const uint4*>(sStg + (16 * wv + r) * 72 + 32 * s2 + 8 * grp);
    *reinterpret_cast<uint4*>(rec + R::AQK + (tri_frag(wv, s2) * 64 + ln) * 16) = u;
  }

  // ---- phase 3: Tm = (I + Akk)^-1 ------------------------------------------------
  // 3a: inverse of the unit lower diagonal block I, one column (r) per lane, by
  //     forward substitution: x_i = -sum_{m<i} A[i][m] x_m for i > r, x_r = 1.
  {
    float x[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) x[m] = (m == r) ? 1.f : 0.f;
    const float* A = sAkk + (16 * wv) * SM::AS + 16 * wv;
#pragma unroll
    for (int ii = 1; ii < 16; ++ii) {
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < ii; ++m) acc += A[ii * SM::AS + m] * x[m];
      if (ii > r) x[ii] = -acc;
    }
    if (grp == 0) {
      float* Aw = sAkk + (16 * wv) * SM::AS + 16 * wv;
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) Aw[ii * SM::AS + r] = x[ii];
    }
  }
  __syncthreads();  // B6: diagonal blocks hold D_I

  // 3b: block column J = wv below the diagonal:
  //     Inv_IJ = -D_I sum_{J<=M<I} A_IM Inv_MJ   (Inv_JJ = D_J),
  //     16x16x16 products as four fp32 MFMAs; step kb takes contraction index
  //     4*grp + kb in lane group grp, so a C-layout result feeds the next
  //     product's B operand straight from its registers.
  f32x4 inv[4];
#pragma unroll
  for (int I = 0; I < 4; ++I) inv[I] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    const int J = wv;
#pragma unroll
    for (int I = 1; I < 4; ++I) {
      if (I <= J) continue;
      f32x4 P = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int M = 0; M < 3; ++M) {
        if (M < J || M >= I) continue;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const float a = sAkk[(16 * I + r) * SM::AS + 16 * M + 4 * grp + kb];
          const float b = (M == J) ? sAkk[(16 * J + 4 * grp + kb) * SM::AS + 16 * J + r] : inv[M][kb];
          P = mfma16x4f32(a, b, P);
        }
      }
      f32x4 Q = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float a = sAkk[(16 * I + r) * SM::AS + 16 * I + 4 * grp + kb];
        Q = mfma16x4f32(a, P[kb], Q);
      }
      inv[I] = -Q;
    }
  }
  __syncthreads();  // B7: every read of the Akk blocks is done
  {
    const int J = wv;
#pragma unroll
    for (int I = 1; I < 4; ++I) {
      if (I <= J) continue;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sAkk[(16 * I + 4 * grp + rr) * SM::AS + 16 * J + r] = inv[I][rr];
    }
  }
  __syncthreads();  // B8: Tm complete

  // ---- phase 4: TmB = Tm diag(beta) record fragments; w = TmB (k exp(Gam)) -------
  bf16x8 TB[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    if (s2 >= tri_steps(wv)) continue;
    const int row = 16 * wv + r, c0 = 32 * s2 + 8 * grp;
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = sAkk[row * SM::AS + c0 + e] * sBeta[c0 + e];
    const uint4 u = pack8(t);
    TB[s2] = as_frag(u);
    *reinterpret_cast<uint4*>(rec + R::TMB + (tri_frag(wv, s2) * 64 + ln) * 16) = u;
  }
#pragma unroll
  for (int nt = 0; nt < K / 16; ++nt) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const int d = 16 * nt + r;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      if (s2 >= tri_steps(wv)) continue;
      const uint4 u = *reinterpret_cast<const uint4*>(sKdT + d * SM::TS + tcol(32 * s2 + 8 * grp, d));
      acc = mfma16x32(TB[s2], as_frag(u), acc);
    }
    // stage -w, C layout: row 16I + 4grp + rr, column d
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) sStg[(16 * wv + 4 * grp + rr) * SM::STG_S + d] = f2bf(-acc[rr]);
  }
  __syncthreads();  // B9
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint4 u = *reinterpret_cast<const uint4*>(sStg + (16 * wv + r) * SM::STG_S + 32 * s + 8 * grp);
    *reinterpret_cast<uint4*>(rec + R::WN + ((wv * S + s) * 64 + ln) * 16) = u;
  }
}

// -------------------------------------------------------- debug unpack
// Record fragments -> plain row-major tensors (one workgroup per record).
template <int K>
__global__ __launch_bounds__(NTHREADS) void unpack_kernel(Params p, int n_items, uint16_t* qg,
                                                          uint16_t* w, uint16_t* kg, uint16_t* aqk,
                                                          uint16_t* tmb, float* alpha) {
  using R = Rec<K>;
  constexpr int S = K / 32;
  const int item = blockIdx.x;
  if (item >= n_items) return;
  const int hv = item % p.HV;
  const int64_t gc = item / p.HV;
  ChunkLoc cl;
  if (!locate_chunk(p, gc, cl)) return;
  const uint8_t* rec = p.recs + (gc * p.HV + hv) * (int64_t)R::BYTES;
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63, r = ln & 15, grp = ln >> 4;
  auto tokrow = [&](int t) { return ((int64_t)cl.b * p.T + cl.row0 + t) * p.HV + hv; };
  const int t = 16 * wv + r;
  for (int s = 0; s < S; ++s) {
    const int d0 = 32 * s + 8 * grp;
    if (t < cl.L) {
      const uint4 uq = *reinterpret_cast<const uint4*>(rec + R::QG + ((wv * S + s) * 64 + ln) * 16);
      uint4 uw = *reinterpret_cast<const uint4*>(rec + R::WN + ((wv * S + s) * 64 + ln) * 16);
      uw.x ^= 0x80008000u; uw.y ^= 0x80008000u; uw.z ^= 0x80008000u; uw.w ^= 0x80008000u;
      if (qg) *reinterpret_cast<uint4*>(qg + tokrow(t) * K + d0) = uq;
      if (w) *reinterpret_cast<uint4*>(w + tokrow(t) * K + d0) = uw;
    }
  }
  // kg^T fragments (md, s2): d = 16md + r, tokens 32s2 + 8grp .. +7
  for (int f = wv; f < 2 * (K / 16); f += 4) {
    const int md = f >> 1, s2 = f & 1;
    const uint4 u = *reinterpret_cast<const uint4*>(rec + R::KGT + (f * 64 + ln) * 16);
    const uint16_t* e = reinterpret_cast<const uint16_t*>(&u);
    for (int j = 0; j < 8; ++j) {
      const int tt = 32 * s2 + 8 * grp + j;
      if (kg && tt < cl.L) kg[tokrow(tt) * K + 16 * md + r] = e[j];
    }
  }
  // triangular 64 x 64: zero fragments are not stored
  for (int s2 = 0; s2 < 2; ++s2) {
    const int c0 = 32 * s2 + 8 * grp;
    uint4 ua = make_uint4(0, 0, 0, 0), ut = ua;
    if (s2 < tri_steps(wv)) {
      ua = *reinterpret_cast<const uint4*>(rec + R::AQK + (tri_frag(wv, s2) * 64 + ln) * 16);
      ut = *reinterpret_cast<const uint4*>(rec + R::TMB + (tri_frag(wv, s2) * 64 + ln) * 16);
    }
    if (t < cl.L) {
      if (aqk) *reinterpret_cast<uint4*>(aqk + tokrow(t) * 64 + c0) = ua;
      if (tmb) *reinterpret_cast<uint4*>(tmb + tokrow(t) * 64 + c0) = ut;
    }
  }
  if (alpha) {
    const float* al = reinterpret_cast<const float*>(rec + R::ALPHA);
    for (int idx = tid; idx < cl.L * K; idx += NTHREADS) alpha[tokrow(idx / K) * K + idx % K] = al[idx % K];
  }
}

// ------------------------------------------------------------ launchers
static int padded8(int64_t n) { return (int)((n + 7) / 8 * 8); }

hipError_t launch_chunk_table(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_intra(const Params& p, hipStream_t s) {
  const int64_t items = p.max_chunks * p.HV;
  if (items == 0) return hipSuccess;
  const int grid = padded8(items);
  if (p.K == 128) hipLaunchKernelGGL(intra_kernel<128>, dim3(grid), dim3(NTHREADS), 0, s, p, (int)items);
  else hipLaunchKernelGGL(intra_kernel<64>, dim3(grid), dim3(NTHREADS), 0, s, p, (int)items);
  return hipGetLastError();
}

hipError_t launch_unpack(const Params& p, uint16_t* qg, uint16_t* w, uint16_t* kg, uint16_t* aqk,
                         uint16_t* tmb, float* alpha, hipStream_t s) {
  const int64_t items = p.max_chunks * p.HV;
  if (items == 0) return hipSuccess;
  if (p.K == 128)
    hipLaunchKernelGGL(unpack_kernel<128>, dim3((int)items), dim3(NTHREADS), 0, s, p, (int)items, qg, w,
                       kg, aqk, tmb, alpha);
  else
    hipLaunchKernelGGL(unpack_kernel<64>, dim3((int)items), dim3(NTHREADS), 0, s, p, (int)items, qg, w,
                       kg, aqk, tmb, alpha);
  return hipGetLastError();
}

}  // namespace kda
