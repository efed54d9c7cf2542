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
// and the factors X_i = exp(Gam_i - mu_I), Y_j = exp(mu_I - Gam_j), which give
// the same-block products exp(Gam_i - Gam_j) = X_i Y_j.  A pair of blocks J < I
// meets at P_{J+1}, the cumsum at the end of block J:
//   exp(Gam_i - Gam_j) = X_i * [Y_j exp(tot_J / 2)] * exp(mu_I - P_{J+1}),
// where the bracket equals exp(P_{J+1} - Gam_j) <= 1 and the last factor is <= 1
// as well.  So Aqk/Akk run on bf16 MFMA with two exponentials per element, and a
// cross-block factor that underflows only where the whole product is negligible
// (below exp(-12) once the X_i it meets is counted).  X and Y are bounded by
// exp(8 |g|) (half a block of decay); per-token gates below -10 (natural log) are
// raised to -10 when loaded, which keeps both within exp(+-80), normal in fp32 and
// bf16.  The Gam-referenced outputs are rebuilt from the same factors:
// exp(Gam_i) = X_i exp(mu_I), exp(Gam_last - Gam_i) = Y_i exp(Gam_last - mu_I); where
// one of those second factors underflows the product is below exp(-12) as well.
//
// Chunk 16 (C16): the 64 rows of an item are four chunks of 16.  Only the diagonal
// blocks of Aqk, Akk and Tm exist, every Gam-referenced factor is taken relative to
// its 16-row chunk (exp(Gam_i - P_I) = X_i exp(tot_I / 2), exp(P_{I+1} - Gam_i) =
// Y_i exp(tot_I / 2)), and each 16-row chunk gets its own decay row exp(tot_I).
//
// Wave I owns rows 16I..16I+15 through the gate phase (the Aqk/Akk blocks are then
// shared out evenly, see phase 2); lane
// l = 16g + r holds row 16I + r and the P-order key dims 32s + pidx(g, e)
// (s = 0..K/32-1, e = 0..7), which is at once an MFMA A/B fragment and the qg
// record layout.  Results leave the MFMA C layout directly as record fragments:
// Aqk is computed transposed (operands swapped) and w as w^T = kd^T TmB^T, so a
// lane's accumulator pair already is its P-order fragment; only kg^T and kd^T
// (contractions over tokens) are transposed through LDS: written row-major, read
// back with the gfx950 transpose read.

#include "kda_device.hpp"
#include "kda_internal.hpp"

#include <algorithm>
#include <atomic>

namespace kda {

template <int K>
struct IntraSmem {
  static constexpr int S = K / 32;
  static constexpr int RS = K + 16;                     // row-major [64][K] tile row stride (bf16)
  static constexpr int TOT = 0;                         // float [4][K] block gate totals
  static constexpr int NTAB = 17;                       // gate table rows
  static constexpr int TAB = TOT + 4 * K * 4;           // float [NTAB][K] E, F, c, H tables
  static constexpr int BETA = TAB + NTAB * K * 4;       // float [64]
  static constexpr int KY = BETA + 256;                 // float [3][S][64][8] k Y H, blocks 0..2
  static constexpr int KY_BYTES = 3 * S * 64 * 8 * 4;
  static constexpr int KT = KY + KY_BYTES;              // bf16 [64][RS]: kg
  static constexpr int KDT = KT + 64 * RS * 2;          // bf16 [64][RS]: k exp(Gam)
  static constexpr int X3 = KDT + 64 * RS * 2;          // bf16 [2][S][64 lanes][8]: q X, k X of row block 3
  static constexpr int END0 = X3 + 2 * S * 64 * 16;
  static constexpr int AS = 68;                         // Akk / Tm row stride (fp32)
  static constexpr int AKK_BYTES = 64 * AS * 4;
  static constexpr int AKK = (KY_BYTES >= AKK_BYTES) ? KY : END0;   // reuses k*Y when it fits
  static constexpr int BYTES = (AKK == KY) ? END0 : END0 + AKK_BYTES;
};

struct ChunkLoc {
  int b;
  int64_t row0;  // first row of the chunk within batch row b
  int L;         // valid rows (1..64)
};

// Chunk gc -> (batch row, first row, valid rows).  Returns false when gc is past
// the last chunk (varlen capacity padding) or the chunk table was rejected.
// The varlen table and chunk info come in as read-only, non-aliasing pointers: with
// a uniform chunk index their loads are scalar loads, which wait on their own
// counter, never on the vector stores of the records in flight.
__device__ __forceinline__ bool locate_chunk(const Params& p, const int32_t* __restrict__ tb,
                                             const int2* __restrict__ cinfo, int64_t gc, ChunkLoc& c) {
  if (p.cu == nullptr) {
    int n = (int)(gc / p.NT);
    if (n >= p.B) return false;
    c.b = n;
    c.row0 = (gc - (int64_t)n * p.NT) * BT;
    c.L = (int)min<int64_t>(BT, p.T - c.row0);
    return c.L > 0;
  }
  if (tb[p.N + 1] != 0 || gc >= tb[p.N]) return false;
  const int2 ci = cinfo[gc];   // first row and valid rows, written by the chunk table kernel
  c.b = 0;
  c.row0 = ci.x;
  c.L = ci.y;
  return c.L > 0;
}

// ----------------------------------------------------------- chunk table
// One workgroup: chunk_base[n] = sum_{m<n} ceil(len_m / 64) (the tile_base of the
// FlashKDA walkthrough's sequence-information section), chunk_base[N] = total,
// and an error flag at [N+1] if cu_seqlens is not 0 = cu[0] <= ... <= cu[N] = T;
// optionally the segment table and, per chunk, its first row and valid rows (so the
// intra stage finds a chunk with one load instead of a search over the table), and
// the sequences sorted by chunk count, longest first (ties by index), so that the
// 64-column scan can hand out its longest scans first.
__global__ __launch_bounds__(256) void chunk_table_kernel(const int64_t* cu, int N, int T, int64_t max_chunks,
                                                           int32_t* table, int32_t* counter, int seg_L,
                                                           int64_t max_segs, int32_t* segtab, int2* cinfo,
                                                           int32_t* order) {
  __shared__ int32_t scan[256];
  __shared__ int32_t sscan[256];
  __shared__ int32_t bad_any;
  __shared__ unsigned long long skey[ORDER_MAX_N];   // chunk count << 32 | ~index: larger key first
  const int tid = threadIdx.x;
  if (tid == 0) {
    bad_any = (cu[0] != 0 || cu[N] != T) ? 1 : 0;
    if (counter) *counter = 0;   // work counter of the intra stage
  }
  __syncthreads();
  int32_t running = 0, srunning = 0;
  for (int base = 0; base < N; base += 256) {
    const int n = base + tid;
    int32_t cnt = 0, scnt = 0;
    if (n < N) {
      const int64_t a = cu[n], e = cu[n + 1];
      if (a < 0 || e < a || e > T) atomicOr(&bad_any, 1);
      else cnt = (int32_t)((e - a + BT - 1) / BT);
      scnt = cnt > seg_L ? (cnt + seg_L - 1) / seg_L : 1;   // segments, at least one per sequence
    }
    scan[tid] = cnt;
    sscan[tid] = scnt;
    if (order && n < N) skey[n] = ((unsigned long long)(uint32_t)cnt << 32) | (0xffffffffu - (uint32_t)n);
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int32_t add = tid >= off ? scan[tid - off] : 0;
      const int32_t sadd = tid >= off ? sscan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      sscan[tid] += sadd;
      __syncthreads();
    }
    if (n < N) {
      const int32_t first = running + scan[tid] - cnt;
      table[n] = first;
      if (segtab) segtab[n] = srunning + sscan[tid] - scnt;
      if (cinfo) {   // per chunk: first row, valid rows (a rejected table is never read)
        const int32_t a0 = (int32_t)cu[n], len = (int32_t)(cu[n + 1] - cu[n]);
        for (int j = 0; j < cnt && first + j < max_chunks; ++j)
          cinfo[first + j] = make_int2(a0 + BT * j, min(BT, len - BT * j));
      }
    }
    running += scan[255];
    srunning += sscan[255];
    __syncthreads();
  }
  if (order && N <= 256) {
    // rank of each key among the N distinct keys (one pass over LDS, no sort rounds)
    __syncthreads();
    if (tid < N) {
      const unsigned long long key = skey[tid];
      int rank = 0;
      for (int m = 0; m < N; ++m) rank += skey[m] > key;
      order[rank] = tid;
    }
  } else if (order) {
    // bitonic sort of the keys, descending; padding keys are 0 and sort last
    int P = 1;
    while (P < N) P <<= 1;
    for (int n = N + tid; n < P; n += 256) skey[n] = 0ull;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P; i += 256) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const unsigned long long a = skey[i], b = skey[ixj];
            if (((i & k) == 0) ? (a < b) : (a > b)) {
              skey[i] = b;
              skey[ixj] = a;
            }
          }
        }
        __syncthreads();
      }
    for (int r = tid; r < N; r += 256) order[r] = (int32_t)(0xffffffffu - (uint32_t)(skey[r] & 0xffffffffull));
  }
  if (tid == 0) {
    table[N] = running;
    if (segtab) segtab[N] = srunning;
    table[N + 1] = (bad_any || running > max_chunks || (segtab && srunning > max_segs)) ? 1 : 0;
  }
}

// Fixed length: only the intra stage's work counter needs resetting (a kernel
// rather than a memset, so the sequence can be captured in a graph).
__global__ void prep_kernel(Params p) {
  if (threadIdx.x == 0) *p.counter = 0;
}

// ------------------------------------------------------------ intra kernel
// Lowest per-token gate (natural log), -10, that the gate factoring takes: the factors of a
// 16-row block are bounded by exp(8 |g|) = exp(80), normal in fp32 and bf16 (whose
// smallest normal number is about exp(-87.3)).  Lower gates are raised to it.  That
// changes the decay of such a token from exp(g) to exp(-10) ~ 4.5e-5, i.e. by at most
// 4.5e-5 of the state it multiplies, well below the bf16 resolution of the outputs.
// The floor is applied to the packed bf16 bits: a negative bf16 value of larger
// magnitude has a larger unsigned 16-bit pattern, positive values lie below 0x8000, so
// one unsigned 16-bit min per pair does it (-inf, 0xff80, becomes -10; so does a NaN
// with its sign bit set).
constexpr uint16_t GATE_MIN_BF16 = 0xc120;   // -10.0
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t gate_floor2(uint32_t w) {
  const u16x2 lim = {GATE_MIN_BF16, GATE_MIN_BF16};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, w), lim));
}
#ifndef KDA_INTRA_OCC
#define KDA_INTRA_OCC 2   // workgroups per CU the register budget is sized for
#endif
template <int K, bool C16>
__global__ __launch_bounds__(NTHREADS, KDA_INTRA_OCC) void intra_kernel(Params p, int n_items,
                                                                         const int32_t* __restrict__ tbl,
                                                                         const int2* __restrict__ cinfo) {
  using SM = IntraSmem<K>;
  using R = Rec<K>;
  constexpr int S = SM::S;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SM::BYTES];
  float* sTot = reinterpret_cast<float*>(smem + SM::TOT);
  float* sTab = reinterpret_cast<float*>(smem + SM::TAB);
  float* sBeta = reinterpret_cast<float*>(smem + SM::BETA);
  float* sKY = reinterpret_cast<float*>(smem + SM::KY);
  uint16_t* sKT = reinterpret_cast<uint16_t*>(smem + SM::KT);
  uint4* sX3 = reinterpret_cast<uint4*>(smem + SM::X3);
  float* sAkk = reinterpret_cast<float*>(smem + SM::AKK);

  const int tid = threadIdx.x;
  // wave index via readfirstlane: branches on it stay scalar (an MFMA under a
  // lane-predicated branch would still write every lane)
  const int I = __builtin_amdgcn_readfirstlane(tid >> 6);   // this wave's 16-row block
  const int ln = tid & 63;
  const int r = ln & 15, g = ln >> 4;
  const int i = 16 * I + r;       // this lane's row in the chunk

  // Persistent: the first round of items is blockIdx-based (XCD-remapped), later
  // items are handed out by an atomic ticket counter, so workgroups that run faster
  // take more items.  The q, k, g, beta of the next item are loaded into registers
  // while the current one is computed (phases 2-3).  lane dims for step s, element e:
  // d = 32s + pidx(g, e)
  __shared__ int s_next;
  __shared__ long long s_nrow;   // first token row of s_next's chunk (batch row folded in)
  __shared__ int s_nlen;         // its valid rows; 0 when there is nothing to do
  uint4 nq[S], nk[S], ng[S];
  uint32_t nb = 0;   // raw bf16 bits: converting here would wait for the loads
  // Location of item `it`: first token row and valid rows (0 past the last item, for
  // varlen capacity padding and for a rejected table).
  auto locate_item = [&](int it, int64_t& row, int& len) {
    it = __builtin_amdgcn_readfirstlane(it);
    ChunkLoc c;
    const bool ok = it < n_items && locate_chunk(p, tbl, cinfo, it / p.HV, c);
    row = ok ? (int64_t)c.b * p.T + c.row0 : 0;
    len = ok ? c.L : 0;
  };
  // Next ticket and its location, by thread 0.  Varlen locations are table loads;
  // made here, right after the ticket atomic (whose result is awaited anyway), they
  // never make the item loads wait for the record stores still in flight.
  auto draw_ticket = [&]() {
    if (tid == 0) {
      const int t = (int)gridDim.x + atomicAdd(p.counter, 1);
      int64_t row;
      int len;
      locate_item(t, row, len);
      s_next = t;
      s_nrow = row;
      s_nlen = len;
    }
  };
  // one input of item `it` at (row, len): 0 = q, 1 = k, 2 = g and beta
  auto fetch_part = [&](int it, int64_t row0, int len, int part) {
    const int h = it % p.HV;
    const bool valid = i < len;
    const int64_t tk = valid ? row0 + i : 0;
    const uint16_t* row = part == 0 ? p.q + (tk * p.HQK + h / (p.HV / p.HQK)) * K
                        : part == 1 ? p.k + (tk * p.HQK + h / (p.HV / p.HQK)) * K
                                    : p.g + (tk * p.HV + h) * K;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int lo = 32 * s + 4 * g, hi = lo + 16;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (valid) {
        const uint2 a0 = *reinterpret_cast<const uint2*>(row + lo), a1 = *reinterpret_cast<const uint2*>(row + hi);
        u = make_uint4(a0.x, a0.y, a1.x, a1.y);
      }
      if (part == 0) nq[s] = u;
      else if (part == 1) nk[s] = u;
      else ng[s] = u;
    }
    if (part == 2) {
      // rows past the chunk get beta = 0: the bf16 bits of 0, or of -inf as a logit
      nb = (p.flags & FLAG_BETA_LOGITS) ? 0xff80u : 0u;
      if (valid) nb = p.beta[tk * p.HV + h];
    }
  };
  auto fetch = [&](int it, int64_t row0, int len) {
    fetch_part(it, row0, len, 0);
    fetch_part(it, row0, len, 1);
    fetch_part(it, row0, len, 2);
  };
  int item = xcd_remap(blockIdx.x, gridDim.x);
  int cur_len;   // valid rows of `item`
  {
    int64_t row;
    locate_item(item, row, cur_len);
    fetch(item, row, cur_len);
  }
  draw_ticket();
  __syncthreads();
  while (item < n_items) {
  // written before the last barrier; rewritten only after B8
  const int next = __builtin_amdgcn_readfirstlane(s_next);
  const int64_t next_row = s_nrow;
  const int next_len = __builtin_amdgcn_readfirstlane(s_nlen);
  const int hv = item % p.HV;
  const int64_t gc = item / p.HV;
  const bool live = cur_len > 0;   // uniform over the workgroup
  uint4 uqs[S], uks[S];   // q, k kept packed (bf16) until used
  float gl[S][8];
  float bt;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    uqs[s] = nq[s];
    uks[s] = nk[s];
    unpack8(make_uint4(gate_floor2(ng[s].x), gate_floor2(ng[s].y), gate_floor2(ng[s].z), gate_floor2(ng[s].w)), gl[s]);
  }
  bt = bf2f((uint16_t)nb);
  if (p.flags & FLAG_BETA_LOGITS)   // FlashKDA's fused sigmoid: 1 / (1 + e^-x), exact 0 and 1 at -inf, +inf
    bt = 1.f / (1.f + __builtin_amdgcn_exp2f(-LOG2E * bt));
  if (!live) {   // varlen capacity padding or rejected table: nothing to write
    fetch(next, next_row, next_len);
    __syncthreads();   // every thread has read s_next
    draw_ticket();
    __syncthreads();
    item = next;
    cur_len = next_len;
    continue;
  }
  uint8_t* rec = p.recs + rec_index(hv, gc, p.HV) * (int64_t)R::BYTES;
  if (g == 0) sBeta[i] = bt;

  // in-block inclusive cumsum over the 16 rows (lanes r = 0..15 of a DPP row)
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) gl[s][e] = row_inclusive_scan(gl[s][e]);
  if (r == 15) {
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) sTot[I * K + 32 * s + pidx(g, e)] = gl[s][e];
  }
  __syncthreads();  // B1: block totals

  // tables, per key dim d (natural-log sums, exp2 of log2e-scaled arguments):
  //   rows 0..3   E_I = exp(mu_I)              mu_I = P_I + tot_I / 2, P_I = sum_{J<I} tot_J
  //   rows 4..7   F_I = exp(Gam_last - mu_I)
  //   rows 8..13  c_IJ = exp(mu_I - P_{J+1}), pair (I,J) -> 8 + I(I-1)/2 + J
  //   rows 14..16 H_J = exp(tot_J / 2), so that Y_j H_J = exp(P_{J+1} - Gam_j)
  // every argument is <= 0 except the midpoint offsets folded into X and Y.  Chunk 16:
  // rows 0..7 are exp(tot_I / 2) (the gate restarts at every 16-row chunk), rows 8..16
  // are not read, and each 16-row chunk's decay row exp(tot_I) is stored.
  {
    constexpr int STEP = NTHREADS / K;            // table rows per pass (2 or 4)
    const int d = tid % K, r0 = tid / K;          // r0 is uniform over a wave (64 divides K)
    const float t0 = sTot[d], t1 = sTot[K + d], t2 = sTot[2 * K + d], t3 = sTot[3 * K + d];
    const float m0 = 0.5f * t0, m1 = t0 + 0.5f * t1, m2 = t0 + t1 + 0.5f * t2, m3 = t0 + t1 + t2 + 0.5f * t3;
    const float P1 = t0, P2 = t0 + t1, P3 = t0 + t1 + t2;
    const float G = t0 + t1 + t2 + t3;
    const float h0 = 0.5f * t0, h1 = 0.5f * t1, h2 = 0.5f * t2, h3 = 0.5f * t3;
    const float arg[SM::NTAB] = {C16 ? h0 : m0, C16 ? h1 : m1, C16 ? h2 : m2, C16 ? h3 : m3,
                                 C16 ? h0 : G - m0, C16 ? h1 : G - m1, C16 ? h2 : G - m2, C16 ? h3 : G - m3,
                                 m1 - P1, m2 - P1, m2 - P2, m3 - P1, m3 - P2, m3 - P3,
                                 h0, h1, h2};
#pragma unroll
    for (int row = 0; row < SM::NTAB; ++row)
      if (row % STEP == r0) sTab[row * K + d] = __builtin_amdgcn_exp2f(LOG2E * arg[row]);
    if (C16) {
      const float tt[4] = {t0, t1, t2, t3};
#pragma unroll
      for (int J = 0; J < 4; ++J)
        if (J % STEP == r0) reinterpret_cast<float*>(rec + alpha16_off<K>(J))[d] = __builtin_amdgcn_exp2f(LOG2E * tt[J]);
    } else if (r0 == 0) {
      reinterpret_cast<float*>(rec + R::ALPHA)[d] = __builtin_amdgcn_exp2f(LOG2E * G);
    }
  }
  __syncthreads();  // B2: tables

  // Row-major [64][K] tiles of kg and of k exp(Gam) (two tiles, so that writing the
  // second needs no barrier after the reads of the first): lane (g, r) writes row i
  // at its P-order dims, 8 bytes at a time.  The row stride of K + 16 elements starts
  // eight consecutive rows on eight different groups of 8 banks.
  uint8_t* const kt_row = reinterpret_cast<uint8_t*>(sKT) + (i * SM::RS + 4 * g) * 2;   // row i, dims 4g..
  // transpose-read lane address: lane (b, j, a) reads row 4b + j, columns 4a..4a+3
  const uint8_t* const kt_tr = reinterpret_cast<const uint8_t*>(sKT) +
                               ((4 * (ln >> 4) + ((ln >> 2) & 3)) * SM::RS + 4 * (ln & 3)) * 2;
  // P-order fragment of the transpose of tile `tile` (byte offset from the kg tile):
  // key dims dim0.., tokens tok0..
  auto kt_frag = [&](int tok0, int dim0, int tile = 0) {
    const uint2 lo = lds_tr8(kt_tr + tile + (tok0 * SM::RS + dim0) * 2);
    const uint2 hi = lds_tr8(kt_tr + tile + ((tok0 + 16) * SM::RS + dim0) * 2);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  };
  bf16x8 QX[S], KX[S], KYr[S];
  uint4 KD[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    uint2 pq[2], pk[2], py[2], pg[2], pd[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint2 qw = hf ? make_uint2(uqs[s].z, uqs[s].w) : make_uint2(uqs[s].x, uqs[s].y);
      const uint2 kw = hf ? make_uint2(uks[s].z, uks[s].w) : make_uint2(uks[s].x, uks[s].y);
      const float qf[4] = {bflo(qw.x), bfhi(qw.x), bflo(qw.y), bfhi(qw.y)};
      const float kf[4] = {bflo(kw.x), bfhi(kw.x), bflo(kw.y), bfhi(kw.y)};
      float qx[4], kx[4], ky[4], qg[4], kd[4], kgv[4];
      const int d0 = 32 * s + 16 * hf + 4 * g;   // 4 consecutive key dims
      const float4 tot4 = *reinterpret_cast<const float4*>(sTot + I * K + d0);
      const float4 E4 = *reinterpret_cast<const float4*>(sTab + I * K + d0);
      const float4 F4 = *reinterpret_cast<const float4*>(sTab + (4 + I) * K + d0);
      const float tot[4] = {tot4.x, tot4.y, tot4.z, tot4.w};
      const float Ev[4] = {E4.x, E4.y, E4.z, E4.w};
      const float Fv[4] = {F4.x, F4.y, F4.z, F4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = gl[s][4 * hf + e] - 0.5f * tot[e];
        const float X = __builtin_amdgcn_exp2f(LOG2E * x);
        const float Y = __builtin_amdgcn_exp2f(-LOG2E * x);
        qx[e] = qf[e] * X;
        kx[e] = kf[e] * X;
        ky[e] = kf[e] * Y;
        qg[e] = p.scale * qx[e] * Ev[e];
        kd[e] = kx[e] * Ev[e];
        kgv[e] = ky[e] * Fv[e];
      }
      pq[hf] = make_uint2(pack2(qx[0], qx[1]), pack2(qx[2], qx[3]));
      pk[hf] = make_uint2(pack2(kx[0], kx[1]), pack2(kx[2], kx[3]));
      py[hf] = make_uint2(pack2(ky[0], ky[1]), pack2(ky[2], ky[3]));
      pg[hf] = make_uint2(pack2(qg[0], qg[1]), pack2(qg[2], qg[3]));
      pd[hf] = make_uint2(pack2(kd[0], kd[1]), pack2(kd[2], kd[3]));
      *reinterpret_cast<uint2*>(kt_row + (32 * s + 16 * hf) * 2) =
          make_uint2(pack2(kgv[0], kgv[1]), pack2(kgv[2], kgv[3]));   // kg, row-major
      if (I < 3) {   // k exp(P_{I+1} - Gam), the cross-block operand of the later row blocks
        const float4 H4 = *reinterpret_cast<const float4*>(sTab + (14 + I) * K + d0);
        reinterpret_cast<float4*>(sKY + ((I * S + s) * 64 + ln) * 8)[hf] =
            make_float4(ky[0] * H4.x, ky[1] * H4.y, ky[2] * H4.z, ky[3] * H4.w);
      }
    }
    QX[s] = as_frag(make_uint4(pq[0].x, pq[0].y, pq[1].x, pq[1].y));
    KX[s] = as_frag(make_uint4(pk[0].x, pk[0].y, pk[1].x, pk[1].y));
    if (I == 3) {   // wave 0 computes row block 3's first Aqk / Akk fragment pair
      sX3[s * 64 + ln] = make_uint4(pq[0].x, pq[0].y, pq[1].x, pq[1].y);
      sX3[(S + s) * 64 + ln] = make_uint4(pk[0].x, pk[0].y, pk[1].x, pk[1].y);
    }
    KYr[s] = as_frag(make_uint4(py[0].x, py[0].y, py[1].x, py[1].y));
    KD[s] = make_uint4(pd[0].x, pd[0].y, pd[1].x, pd[1].y);
    store_stream(rec + R::QG + ((I * S + s) * 64 + ln) * 16, make_uint4(pg[0].x, pg[0].y, pg[1].x, pg[1].y));
  }
  __syncthreads();  // B3: k*Y blocks, kg^T

  // ---- phase 2: kg^T record; (k exp(Gam))^T; transposed Aqk / Akk of block row I --
  for (int f = I; f < 2 * (K / 16); f += 4) {
    const int md = f >> 1, s2 = f & 1;
    store_stream(rec + R::KGT + (f * 64 + ln) * 16, kt_frag(32 * s2, 16 * md));
  }
  // The next item's inputs load in three parts spread over phases 2-3 (g here, q
  // after B5, k after B6): issued at once they waited about 6k cycles per item
  // for queue space behind this item's record stores.
  fetch_part(next, next_row, next_len, 2);   // g and beta of the next item
#pragma unroll
  for (int s = 0; s < S; ++s) {   // k exp(Gam), row-major
    *reinterpret_cast<uint2*>(kt_row + (SM::KDT - SM::KT) + (32 * s) * 2) = make_uint2(KD[s].x, KD[s].y);
    *reinterpret_cast<uint2*>(kt_row + (SM::KDT - SM::KT) + (32 * s + 16) * 2) = make_uint2(KD[s].z, KD[s].w);
  }
  // C = (k Y H c) (q X)^T: lane holds [j = 16J + 4g + rr][i = 16I + r], i.e. row i of
  // Aqk / Akk at columns 16J + 4g + rr -- already the P-order A fragment of the
  // inter kernel's Aqk v' product.  Block J = I uses this wave's own k Y (no H, c).
  // The ten nonzero 16x16 blocks (J <= I) are shared out as fragment pairs (row block
  // Ib, columns 32 s2..): wave 0 takes (0, 0) and (3, 0), wave 1 (1, 0), wave 2 (2, 0)
  // and (2, 1), wave 3 (3, 1) -- at most three blocks per wave instead of four for
  // wave 3.  Row block 3's q X and k X reach wave 0 through LDS, its beta from sBeta.
  auto job = [&](const int Ib, const int s2, f32x4* vko) {
    const bool own = Ib == I;
    const float bti = own ? bt : sBeta[16 * Ib + r];
    f32x4 vq[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int J = 2 * s2 + h;
      f32x4 aq = f32x4{0.f, 0.f, 0.f, 0.f}, ak = aq;
      const bool cross = !C16 && J < Ib;   // chunk 16: only the diagonal blocks exist
      if (J == Ib || cross) {
        const int pr = 8 + Ib * (Ib - 1) / 2 + J;   // c_IJ table row (J < Ib)
#pragma unroll
        for (int s = 0; s < S; ++s) {
          bf16x8 A;
          if (J == Ib) {
            A = KYr[s];   // only when own
          } else {
            const float4* src = reinterpret_cast<const float4*>(sKY + ((J * S + s) * 64 + ln) * 8);
            const float4 a0 = src[0], a1 = src[1];
            const float* c = sTab + pr * K + 32 * s;
            const float4 c0 = *reinterpret_cast<const float4*>(c + 4 * g);
            const float4 c1 = *reinterpret_cast<const float4*>(c + 16 + 4 * g);
            const float b[8] = {a0.x * c0.x, a0.y * c0.y, a0.z * c0.z, a0.w * c0.w,
                                a1.x * c1.x, a1.y * c1.y, a1.z * c1.z, a1.w * c1.w};
            A = as_frag(pack8(b));
          }
          const bf16x8 bq = own ? QX[s] : as_frag(sX3[s * 64 + ln]);
          const bf16x8 bk = own ? KX[s] : as_frag(sX3[(S + s) * 64 + ln]);
          aq = mfma16x32(A, bq, aq);
          ak = mfma16x32(A, bk, ak);
        }
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int j = 4 * g + rr;   // column within block J
        vq[h][rr] = (cross || (J == Ib && j <= r)) ? p.scale * aq[rr] : 0.f;
        vko[h][rr] = (cross || (J == Ib && j < r)) ? -bti * ak[rr] : 0.f;   // -Akk
      }
    }
    store_stream(rec + R::AQK + (tri_frag(Ib, s2) * 64 + ln) * 16, pack_pair(vq[0], vq[1]));
  };
  f32x4 vkA[2], vkB[2];
  if (I == 0) {
    job(0, 0, vkA);
    job(3, 0, vkB);
  } else if (I == 1) {
    job(1, 0, vkA);
  } else if (I == 2) {
    job(2, 0, vkA);
    job(2, 1, vkB);
  } else {
    job(3, 1, vkA);
  }
  __syncthreads();  // B4: every read of k*Y is done (Akk reuses its space)
  auto put_akk = [&](int Ib, int s2, const f32x4* v) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<float4*>(sAkk + (16 * Ib + r) * SM::AS + 16 * (2 * s2 + h) + 4 * g) =
          make_float4(v[h][0], v[h][1], v[h][2], v[h][3]);
  };
  if (I == 0) {
    put_akk(0, 0, vkA);
    put_akk(3, 0, vkB);
  } else if (I == 1) {
    put_akk(1, 0, vkA);
  } else if (I == 2) {
    put_akk(2, 0, vkA);
    put_akk(2, 1, vkB);
  } else {
    put_akk(3, 1, vkA);
  }
  __syncthreads();  // B5: Akk and (k exp(Gam))^T complete
  fetch_part(next, next_row, next_len, 0);   // q of the next item

  // ---- phase 3: Tm = (I + Akk)^-1 ------------------------------------------------
  // 3a: inverse of the unit lower diagonal block I + N (N strictly lower, so
  //     N^16 = 0): (I + N)^-1 = sum_k (-N)^k = (I - N)(I + N^2)(I + N^4)(I + N^8).
  //     All operands stay in the 16x16 C layout.  With the contraction index of
  //     step kb = 4g + kb in lane group g, the C layout of X^T is exactly the A
  //     operand of X and the C layout of Y the B operand of Y, so a product needs
  //     X^T and Y in C layout and returns X Y in C layout.  The powers of N
  //     commute with the partial products, which are built as D <- D + N^(2^j) D.
  //     The Akk blocks sit in LDS negated (the sign rides on beta when they leave
  //     the accumulators): the first factor I - N is then I plus the stored block,
  //     the even powers do not see the sign, and in 3b the minus of the recursion
  //     is already in the stored A_MP.
  {
    auto mm = [&](const f32x4& xt, const f32x4& y) {
      f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) c = mfma16x4f32(xt[kb], y[kb], c);
      return c;
    };
    const float* A = sAkk + (16 * I) * SM::AS + 16 * I;
    f32x4 N, NT;   // lane: N[4g+e][r] and N[r][4g+e]
#pragma unroll
    for (int e = 0; e < 4; ++e) N[e] = A[(4 * g + e) * SM::AS + r];
    {
      const float4 t = *reinterpret_cast<const float4*>(A + r * SM::AS + 4 * g);
      NT = f32x4{t.x, t.y, t.z, t.w};
    }
    const f32x4 N2 = mm(NT, N), N2T = mm(N, NT);
    const f32x4 N4 = mm(N2T, N2), N4T = mm(N2, N2T);
    const f32x4 N8T = mm(N4, N4T);
    f32x4 D;
#pragma unroll
    for (int e = 0; e < 4; ++e) D[e] = (4 * g + e == r ? 1.f : 0.f) + N[e];   // N holds -Akk
    D += mm(N2T, D);
    D += mm(N4T, D);
    D += mm(N8T, D);
    float* Aw = sAkk + (16 * I) * SM::AS + 16 * I;
#pragma unroll
    for (int e = 0; e < 4; ++e) Aw[(4 * g + e) * SM::AS + r] = D[e];
  }
  __syncthreads();  // B6: diagonal blocks hold D_I
  fetch_part(next, next_row, next_len, 1);   // k of the next item

  // 3b: block column J = I below the diagonal:
  //     Inv_MJ = -D_M sum_{J<=P<M} A_MP Inv_PJ   (Inv_JJ = D_J),
  //     16x16x16 products as four fp32 MFMAs; step kb takes contraction index
  //     4g + kb in lane group g, so a C-layout result feeds the next product's B
  //     operand straight from its registers.
  //     Chunk 16: Akk is block diagonal, so these blocks are zero and stay zero in LDS.
  f32x4 inv[4];
#pragma unroll
  for (int M = 0; M < 4; ++M) inv[M] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (!C16) {
    const int J = I;
#pragma unroll
    for (int M = 1; M < 4; ++M) {
      if (M <= J) continue;
      f32x4 P = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int Q = 0; Q < 3; ++Q) {
        if (Q < J || Q >= M) continue;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const float a = sAkk[(16 * M + r) * SM::AS + 16 * Q + 4 * g + kb];
          const float b = (Q == J) ? sAkk[(16 * J + 4 * g + kb) * SM::AS + 16 * J + r] : inv[Q][kb];
          P = mfma16x4f32(a, b, P);
        }
      }
      f32x4 D = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float a = sAkk[(16 * M + r) * SM::AS + 16 * M + 4 * g + kb];
        D = mfma16x4f32(a, P[kb], D);
      }
      inv[M] = D;   // the Akk blocks are stored negated
    }
  }
  __syncthreads();  // B7: every read of the Akk blocks is done
#pragma unroll
  for (int M = 1; M < 4; ++M) {
    if (C16 || M <= I) continue;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) sAkk[(16 * M + 4 * g + rr) * SM::AS + 16 * I + r] = inv[M][rr];
  }
  __syncthreads();  // B8: Tm complete

  // ---- phase 4: TmB = Tm diag(beta) fragments; w^T = (k exp(Gam))^T TmB^T ----------
  // Chunk 16: fragment (I, 0) of row blocks 2 and 3 is zero (block diagonal); its record
  // slot holds the decay rows instead, and its products are skipped.
  bf16x8 TBn[2];   // -TmB: the w products then leave -w, the WN record, directly
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    if (s2 >= tri_steps(I) || (C16 && I >= 2 && s2 == 0)) continue;
    const float* trow = sAkk + i * SM::AS + 32 * s2;
    const float* brow = sBeta + 32 * s2;
    const float4 t0 = *reinterpret_cast<const float4*>(trow + 4 * g);
    const float4 t1 = *reinterpret_cast<const float4*>(trow + 16 + 4 * g);
    const float4 b0 = *reinterpret_cast<const float4*>(brow + 4 * g);
    const float4 b1 = *reinterpret_cast<const float4*>(brow + 16 + 4 * g);
    const float t[8] = {t0.x * b0.x, t0.y * b0.y, t0.z * b0.z, t0.w * b0.w,
                        t1.x * b1.x, t1.y * b1.y, t1.z * b1.z, t1.w * b1.w};
    const uint4 u = pack8(t);
    TBn[s2] = as_frag(make_uint4(u.x ^ 0x80008000u, u.y ^ 0x80008000u, u.z ^ 0x80008000u, u.w ^ 0x80008000u));
    store_stream(rec + R::TMB + (tri_frag(I, s2) * 64 + ln) * 16, u);
  }
  // C[d][t] = sum_t' kd[t'][d] TmB[t][t'] = w[t][d]: lane holds w row 16I + r at
  // key dims 16md + 4g + rr, so tile pairs (md = 2s, 2s+1) form WN fragment (I, s).
#pragma unroll
  for (int s = 0; s < S; ++s) {
    f32x4 acc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        if (s2 >= tri_steps(I) || (C16 && I >= 2 && s2 == 0)) continue;
        acc[h] = mfma16x32(as_frag(kt_frag(32 * s2, 16 * (2 * s + h), SM::KDT - SM::KT)), TBn[s2], acc[h]);
      }
    }
    store_stream(rec + R::WN + ((I * S + s) * 64 + ln) * 16, pack_pair(acc[0], acc[1]));
  }
  draw_ticket();     // ticket (and location) for the item after next
  __syncthreads();  // B9: phase-4 reads of Tm, beta and (k exp(Gam))^T are done; s_next visible
  item = next;
  cur_len = next_len;
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
  if (!locate_chunk(p, p.table, p.cinfo, gc, cl)) return;
  const uint8_t* rec = p.recs + rec_index(hv, gc, p.HV) * (int64_t)R::BYTES;
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63, r = ln & 15, g = ln >> 4;
  auto tokrow = [&](int t) { return ((int64_t)cl.b * p.T + cl.row0 + t) * p.HV + hv; };
  const int t = 16 * wv + r;
  for (int s = 0; s < S; ++s) {
    const uint4 uq = *reinterpret_cast<const uint4*>(rec + R::QG + ((wv * S + s) * 64 + ln) * 16);
    const uint4 uw = *reinterpret_cast<const uint4*>(rec + R::WN + ((wv * S + s) * 64 + ln) * 16);
    const uint16_t* eq = reinterpret_cast<const uint16_t*>(&uq);
    const uint16_t* ew = reinterpret_cast<const uint16_t*>(&uw);
    if (t < cl.L)
      for (int e = 0; e < 8; ++e) {
        const int d = 32 * s + pidx(g, e);
        if (qg) qg[tokrow(t) * K + d] = eq[e];
        if (w) w[tokrow(t) * K + d] = ew[e] ^ 0x8000;
      }
  }
  // kg^T fragments (md, s2): d = 16md + r, tokens 32s2 + pidx(g, e)
  for (int f = wv; f < 2 * (K / 16); f += 4) {
    const int md = f >> 1, s2 = f & 1;
    const uint4 u = *reinterpret_cast<const uint4*>(rec + R::KGT + (f * 64 + ln) * 16);
    const uint16_t* e = reinterpret_cast<const uint16_t*>(&u);
    for (int j = 0; j < 8; ++j) {
      const int tt = 32 * s2 + pidx(g, j);
      if (kg && tt < cl.L) kg[tokrow(tt) * K + 16 * md + r] = e[j];
    }
  }
  // triangular 64 x 64: zero fragments are not stored
  for (int s2 = 0; s2 < 2; ++s2) {
    uint4 ua = make_uint4(0, 0, 0, 0), ut = ua;
    if (s2 < tri_steps(wv)) {
      ua = *reinterpret_cast<const uint4*>(rec + R::AQK + (tri_frag(wv, s2) * 64 + ln) * 16);
      ut = *reinterpret_cast<const uint4*>(rec + R::TMB + (tri_frag(wv, s2) * 64 + ln) * 16);
    }
    const uint16_t* ea = reinterpret_cast<const uint16_t*>(&ua);
    const uint16_t* et = reinterpret_cast<const uint16_t*>(&ut);
    if (t < cl.L)
      for (int e = 0; e < 8; ++e) {
        const int c = 32 * s2 + pidx(g, e);
        if (aqk) aqk[tokrow(t) * 64 + c] = ea[e];
        if (tmb) tmb[tokrow(t) * 64 + c] = et[e];
      }
  }
  if (alpha) {
    const float* al = reinterpret_cast<const float*>(rec + R::ALPHA);
    for (int idx = tid; idx < cl.L * K; idx += NTHREADS) alpha[tokrow(idx / K) * K + idx % K] = al[idx % K];
  }
}

// ------------------------------------------------------------ launchers
static int padded8(int64_t n) { return (int)((n + 7) / 8 * 8); }

hipError_t launch_chunk_table(const int64_t* cu, int N, int T, int64_t max_chunks, int32_t* table,
                              int32_t* counter, int seg_L, int64_t max_segs, int32_t* segtab, int2* cinfo,
                              int32_t* order, hipStream_t s) {
  if (order && N > ORDER_MAX_N) return hipErrorInvalidValue;
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, s, cu, N, T, max_chunks, table, counter,
                     seg_L, max_segs, segtab, cinfo, order);
  return hipGetLastError();
}

// Compute units of the current device, cached per device id.  The cache entries are
// atomics (relaxed): threads that call the library at once may each query the count,
// and every one stores the same value.
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_prep(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL(prep_kernel, dim3(1), dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_intra(const Params& p, hipStream_t s) {
  const int64_t items = p.max_chunks * p.HV;
  if (items == 0) return hipSuccess;
  // persistent grid: KDA_INTRA_OCC resident workgroups per CU, each looping over items
  const int grid = padded8(std::min<int64_t>(items, (int64_t)device_cus() * KDA_INTRA_OCC));
  const dim3 gd(grid), bd(NTHREADS);
  if (p.K == 128) {
    if (p.c16) hipLaunchKernelGGL((intra_kernel<128, true>), gd, bd, 0, s, p, (int)items, p.table, p.cinfo);
    else hipLaunchKernelGGL((intra_kernel<128, false>), gd, bd, 0, s, p, (int)items, p.table, p.cinfo);
  } else {
    if (p.c16) hipLaunchKernelGGL((intra_kernel<64, true>), gd, bd, 0, s, p, (int)items, p.table, p.cinfo);
    else hipLaunchKernelGGL((intra_kernel<64, false>), gd, bd, 0, s, p, (int)items, p.table, p.cinfo);
  }
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
