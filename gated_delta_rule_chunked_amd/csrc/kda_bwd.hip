// kda_bwd.hip -- reverse state scan of the KDA chunked backward for gfx950.
//
// The stage the kernel-fun page "kernel_fun/kda/_kernels/bwd_dhu.py" documents in
// its module docstring.  Given the gradient do of o and dht of the final state,
// and the forward's chunk operands qg = q exp2(g2), kg = k exp2(g2_last - g2), w
// and the chunk-local log2 gate cumsum g2, one workgroup per (sequence, value
// head, 16-column value tile) walks the chunks newest first with dh [K, 16] in
// fp32 registers, starting from dht (or 0):
//   dhc[c] = dh                                  gradient of the state after chunk c
//   dv2    = kg dh + dv                          [64, 16]; dv is the local dL/dv'
//   dh    <- diag(exp2 gd) dh + scale qg^T do - w^T dv2     gd = g2 at the last row
// and dh0 = dh after the oldest chunk.
//
// Eight waves in three roles, one workgroup barrier per chunk (the forward scan's
// arrangement):
//   wave 0 (state wave): dh in the C layout of 16x16 MFMA tiles and the three
//     products of a chunk on bf16 MFMA: DV = kg dh (pairs of dh tiles are its B
//     operand, P-order), QD = qg^T do and WD = w^T dv2 (pairs of dv2 tiles are its B
//     operand).  The two token contractions read row-major LDS tiles through the
//     transpose read (lds_tr8), so no operand is ever transposed by a store.
//   waves 1-4 (helper waves): stage the do and dv tiles and the decay vector of
//     the next chunk (from a register ring fed five phases ahead), and store dv2
//     and the checkpoint of the previous chunk, which the state wave publishes in
//     LDS in its C layout and the transpose read turns back into row segments.
//   waves 5-7 (loader waves): one K-wide operand each (kg, qg, w); three chunks in
//     flight in a register ring of plain 16-byte loads, copied row-major into the
//     free slot of a two-slot LDS ring.
// Phase p (between barriers p-1 and p) is the p-th chunk from the end: the state
// wave runs it, the helpers store the outputs of phase p-1 and stage phase p+1,
// the loaders stage phase p+1 and fetch phase p+3.

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

constexpr int BWD_THREADS = 512;
constexpr int BWD_LD_RING = 3;    // chunks of K-wide operands in flight per loader wave
constexpr int BWD_OUT_RING = 6;   // helper-wave ring (phases); a multiple of BWD_LD_RING

template <int K>
struct BwdSmem {
  // Row-major [64][K] tiles padded by 16 elements: eight consecutive rows then
  // start on eight different groups of 8 banks, so the transpose reads of 16 rows
  // x 32 bytes and the 16-byte row writes run at full LDS rate.
  static constexpr int RS = K + 16;                 // row stride (bf16)
  static constexpr int KT_BYTES = BT * RS * 2;
  static constexpr int KG = 0;                      // kg [64][K]
  static constexpr int QG = KT_BYTES;               // qg [64][K]
  static constexpr int W = 2 * KT_BYTES;            // w  [64][K]
  static constexpr int DO = 3 * KT_BYTES;           // do [64][16] (unpadded: 8 rows cover the banks)
  static constexpr int DV = DO + BT * BV * 2;       // dv [64][16]
  static constexpr int ALPHA = DV + BT * BV * 2;    // exp2(gd), fp32 [K]
  static constexpr int STAGE = ALPHA + K * 4;       // one slot of the ring
  // published outputs of a chunk, C layout (64 lanes x 8 bytes per 16x16 tile):
  // dv2 (4 tiles, bf16), then the checkpoint (K/16 tiles: bf16, or the high and
  // low 16-bit halves of fp32 as two sets of tiles)
  static constexpr int PDV2 = 0;
  static constexpr int PDH = 4 * 512;
  static constexpr int PUB_BYTES = PDH + 2 * (K / 16) * 512;
  static constexpr int PUB = 2 * STAGE;             // two buffers
  static constexpr int BYTES = PUB + 2 * PUB_BYTES;
  static_assert(BYTES <= 160 * 1024, "fits the LDS of one CU");
  static_assert((RS * 2) % 16 == 0 && STAGE % 16 == 0, "16-byte aligned rows and slots");
  static_assert(BWD_OUT_RING % BWD_LD_RING == 0, "one phase count serves every role");
};

template <int K>
__global__ __launch_bounds__(BWD_THREADS, 1) void bwd_dhu_kernel(BwdParams p, int n_items) {
  using SM = BwdSmem<K>;
  constexpr int S = K / 32, ND = K / 16, PF = BWD_OUT_RING - 1;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SM::BYTES];

  // With the longest-first order (varlen) every workgroup of the grid is mapped to a
  // (sequence rank, head) unit in dispatch order, a unit's tiles following in
  // consecutive rounds of eight on one XCD; otherwise items are XCD-remapped.
  const bool lpt = p.order != nullptr;
  const int item = lpt ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
  if (lpt) n_items = (int)gridDim.x;
  if (item >= n_items) return;
  const int NVT = p.V / BV;
  int vt, hv, n;
  bool unit_ok = true;
  if (lpt) {
    const int rnd = item >> 3;
    const int64_t u = (int64_t)(rnd / NVT) * 8 + (item & 7);
    unit_ok = u < (int64_t)p.N * p.HV;
    vt = rnd % NVT;
    hv = unit_ok ? (int)(u % p.HV) : 0;
    n = unit_ok ? p.order[u / p.HV] : 0;
    if ((unsigned)n >= (unsigned)p.N) unit_ok = false, n = 0;   // never for an order the chunk table wrote
  } else {
    vt = item % NVT;
    hv = (item / NVT) % p.HV;
    n = item / (NVT * p.HV);
  }
  const int tid = threadIdx.x, ln = tid & 63, r = ln & 15, g = ln >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar role branches
  const bool state_bf16 = p.flags & FLAG_STATE_BF16;

  SeqLoc sq;
  if (p.cu == nullptr) {
    sq.b = n; sq.bos = 0; sq.len = p.T; sq.cbase = (int64_t)n * p.NT;
  } else {
    if (p.table[p.N + 1] != 0) {
      // rejected cu_seqlens: poison this tile's dh0 and, grid-strided, all of dv2
      const float qnan = __builtin_nanf("");
      if (p.dh0 && unit_ok)
        for (int idx = tid; idx < K * BV; idx += BWD_THREADS)
          store_state(state_bf16, p.dh0, (((int64_t)n * p.HV + hv) * K + idx / BV) * p.V + vt * BV + idx % BV, qnan);
      const int64_t total = (int64_t)p.B * p.T * p.HV * p.V;
      for (int64_t idx = (int64_t)item * BWD_THREADS + tid; idx < total; idx += (int64_t)n_items * BWD_THREADS)
        p.dv2[idx] = 0x7fc0;
      return;
    }
    if (!unit_ok) return;
    sq.b = 0; sq.bos = p.cu[n]; sq.len = (int)(p.cu[n + 1] - p.cu[n]); sq.cbase = p.table[n];
  }
  const int nc = (sq.len + BT - 1) / BT;
  // phases 0..nc (the last only stores the outputs of the oldest chunk), in whole
  // ring turns; every role runs the same count, one barrier each
  const int nphase = (nc + 1 + BWD_OUT_RING - 1) / BWD_OUT_RING * BWD_OUT_RING;
  // first token row of this sequence and value head (row stride HV * width)
  const int64_t row0 = (int64_t)sq.b * p.T + sq.bos;
  // chunk of phase ph (newest first), clamped so the pipeline tail re-reads chunk 0
  auto chunk_of = [&](int ph) { return nc - 1 - min(ph, nc - 1); };

  if (wave == 0) {
    // ============================ state wave ============================
    // dh tile md: lane holds dh[16md + 4g + rr][vt*16 + r], rr = 0..3
    f32x4 dh[ND];
#pragma unroll
    for (int md = 0; md < ND; ++md)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d = 16 * md + 4 * g + rr;
        dh[md][rr] = p.dht ? load_state(state_bf16, p.dht, (((int64_t)n * p.HV + hv) * K + d) * p.V + vt * BV + r) : 0.f;
      }
    // per-lane parts of the LDS addresses
    const int tb = ln >> 4, tj = (ln >> 2) & 3, ta = ln & 3;          // transpose-read source lane
    const int trK = ((4 * tb + tj) * SM::RS + 4 * ta) * 2;            // in a [64][K] tile
    const int tr16 = ((4 * tb + tj) * BV + 4 * ta) * 2;               // in a [64][16] tile
    const int kgA = (r * SM::RS + 4 * g) * 2;                         // A fragment of kg
    const bool dhc_on = p.dhc != nullptr, ckpt_bf16 = p.flags & FLAG_CKPT_BF16;
    barrier_lds();  // S0
    for (int ph = 0; ph < nphase; ++ph) {
      if (ph < nc) {
        const uint8_t* st = smem + (ph & 1) * SM::STAGE;
        uint8_t* pub = smem + SM::PUB + (ph & 1) * SM::PUB_BYTES;
        // dh as the bf16 B operand of DV; published as the checkpoint
        uint2 hb[ND];
#pragma unroll
        for (int md = 0; md < ND; ++md) hb[md] = pack4(dh[md]);
        if (dhc_on) {
          if (ckpt_bf16) {
#pragma unroll
            for (int md = 0; md < ND; ++md) *reinterpret_cast<uint2*>(pub + SM::PDH + (md * 64 + ln) * 8) = hb[md];
          } else {
#pragma unroll
            for (int md = 0; md < ND; ++md) {
              const uint32_t u0 = f2u(dh[md][0]), u1 = f2u(dh[md][1]), u2 = f2u(dh[md][2]), u3 = f2u(dh[md][3]);
              *reinterpret_cast<uint2*>(pub + SM::PDH + (md * 64 + ln) * 8) =
                  make_uint2((u0 >> 16) | (u1 & 0xffff0000u), (u2 >> 16) | (u3 & 0xffff0000u));
              *reinterpret_cast<uint2*>(pub + SM::PDH + ((ND + md) * 64 + ln) * 8) =
                  make_uint2((u0 & 0xffffu) | (u1 << 16), (u2 & 0xffffu) | (u3 << 16));
            }
          }
        }
        // batch 1: dv tiles (C layout, the accumulators' start) and kg A fragments
        uint2 dvi[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) dvi[mb] = lds_tr8(st + SM::DV + tr16 + mb * 16 * BV * 2);
        uint2 kl[4 * S], kh[4 * S];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int s = 0; s < S; ++s) {
            const uint8_t* a = st + SM::KG + kgA + (16 * mb * SM::RS + 32 * s) * 2;
            kl[mb * S + s] = lds8(a);
            kh[mb * S + s] = lds8(a + 32);
          }
        __builtin_amdgcn_sched_barrier(0);
        // DV = kg dh, accumulated onto dv: dv2 in fp32
        f32x4 acc[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[mb] = f32x4{bflo(dvi[mb].x), bfhi(dvi[mb].x), bflo(dvi[mb].y), bfhi(dvi[mb].y)};
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const bf16x8 hbs = cat(hb[2 * s], hb[2 * s + 1]);
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) acc[mb] = mfma16x32(cat(kl[mb * S + s], kh[mb * S + s]), hbs, acc[mb]);
        }
        // batch 2: do B fragments and qg^T A fragments (token contractions, P-order)
        uint2 dol[2], doh[2], ql[2 * ND], qh[2 * ND];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          dol[s2] = lds_tr8(st + SM::DO + tr16 + (32 * s2) * BV * 2);
          doh[s2] = lds_tr8(st + SM::DO + tr16 + (32 * s2 + 16) * BV * 2);
        }
#pragma unroll
        for (int md = 0; md < ND; ++md)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const uint8_t* a = st + SM::QG + trK + ((32 * s2) * SM::RS + 16 * md) * 2;
            ql[md * 2 + s2] = lds_tr8(a);
            qh[md * 2 + s2] = lds_tr8(a + 16 * SM::RS * 2);
          }
        // QD = qg^T do
        f32x4 qd[ND];
#pragma unroll
        for (int md = 0; md < ND; ++md) {
          qd[md] = mfma16x32(cat(ql[md * 2], qh[md * 2]), cat(dol[0], doh[0]), f32x4{0.f, 0.f, 0.f, 0.f});
          qd[md] = mfma16x32(cat(ql[md * 2 + 1], qh[md * 2 + 1]), cat(dol[1], doh[1]), qd[md]);
        }
        // dv2 in bf16: published for the helpers, negated as the B operand of WD
        uint2 vp[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          vp[mb] = pack4(acc[mb]);
          *reinterpret_cast<uint2*>(pub + SM::PDV2 + (mb * 64 + ln) * 8) = vp[mb];
          vp[mb].x ^= 0x80008000u;
          vp[mb].y ^= 0x80008000u;
        }
        __builtin_amdgcn_sched_barrier(0);
        // batch 3: w^T A fragments and the decay
        uint2 wl[2 * ND], wh[2 * ND];
        float4 al[ND];
#pragma unroll
        for (int md = 0; md < ND; ++md)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const uint8_t* a = st + SM::W + trK + ((32 * s2) * SM::RS + 16 * md) * 2;
            wl[md * 2 + s2] = lds_tr8(a);
            wh[md * 2 + s2] = lds_tr8(a + 16 * SM::RS * 2);
          }
#pragma unroll
        for (int md = 0; md < ND; ++md) al[md] = *reinterpret_cast<const float4*>(st + SM::ALPHA + (16 * md + 4 * g) * 4);
        // dh <- diag(alpha) dh + scale QD - w^T dv2
        const bf16x8 vn0 = cat(vp[0], vp[1]), vn1 = cat(vp[2], vp[3]);
#pragma unroll
        for (int md = 0; md < ND; ++md) {
          f32x4 x;
          x[0] = al[md].x * dh[md][0] + p.scale * qd[md][0];
          x[1] = al[md].y * dh[md][1] + p.scale * qd[md][1];
          x[2] = al[md].z * dh[md][2] + p.scale * qd[md][2];
          x[3] = al[md].w * dh[md][3] + p.scale * qd[md][3];
          x = mfma16x32(cat(wl[md * 2], wh[md * 2]), vn0, x);
          dh[md] = mfma16x32(cat(wl[md * 2 + 1], wh[md * 2 + 1]), vn1, x);
        }
      }
      barrier_lds();
    }
    if (p.dh0) {
#pragma unroll
      for (int md = 0; md < ND; ++md)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d = 16 * md + 4 * g + rr;
          store_state(state_bf16, p.dh0, (((int64_t)n * p.HV + hv) * K + d) * p.V + vt * BV + r, dh[md][rr]);
        }
    }
  } else if (wave <= 4) {
    // ============================ helper waves ============================
    const int hw = wave - 1;
    const int otid = tid - 64;                  // 0..255 over the four helper waves
    const int trow = otid >> 2, c4 = 4 * (otid & 3);
    if (nc == 0) {                              // empty sequence: only keep the barrier count
      for (int ph = 0; ph <= nphase; ++ph) barrier_lds();
      return;
    }
    const bool alpha_lane = hw == 0 && ln < K / 4;
    struct Ops {
      uint2 dout, dv;
      float4 g2;
    };
    // operands of phase ph: do / dv row trow of its chunk (clamped into the
    // sequence; rows past the end are zeroed when staged) and g2 at its last row
    auto load = [&](int ph, Ops& op) {
      const int c = chunk_of(ph);
      const int64_t t = row0 + min(c * BT + trow, sq.len - 1);
      const int64_t vo = (t * p.HV + hv) * p.V + vt * BV + c4;
      op.dout = *reinterpret_cast<const uint2*>(p.dout + vo);
      op.dv = p.dv ? *reinterpret_cast<const uint2*>(p.dv + vo) : make_uint2(0, 0);
      if (alpha_lane) {
        const int64_t tl = row0 + min(c * BT + BT, sq.len) - 1;
        op.g2 = *reinterpret_cast<const float4*>(p.g2 + (tl * p.HV + hv) * K + 4 * ln);
      }
    };
    auto stage = [&](int ph, const Ops& op) {
      uint8_t* st = smem + (ph & 1) * SM::STAGE;
      const bool ok = chunk_of(ph) * BT + trow < sq.len;
      *reinterpret_cast<uint2*>(st + SM::DO + (trow * BV + c4) * 2) = ok ? op.dout : make_uint2(0, 0);
      *reinterpret_cast<uint2*>(st + SM::DV + (trow * BV + c4) * 2) = ok ? op.dv : make_uint2(0, 0);
      if (alpha_lane)
        *reinterpret_cast<float4*>(st + SM::ALPHA + 16 * ln) =
            make_float4(__builtin_amdgcn_exp2f(op.g2.x), __builtin_amdgcn_exp2f(op.g2.y),
                        __builtin_amdgcn_exp2f(op.g2.z), __builtin_amdgcn_exp2f(op.g2.w));
    };
    // Un-transposing a published C-layout tile: this lane addresses the slot of
    // C lane (g = ln & 3, r = 4 (ln >> 4) + ((ln >> 2) & 3)) and receives row
    // 16 tile + (ln & 15), columns 4 (ln >> 4) .. +3 of the tile.
    const int src = (16 * (ln & 3) + 4 * (ln >> 4) + ((ln >> 2) & 3)) * 8;
    const int orow = ln & 15, ocol = vt * BV + 4 * (ln >> 4);
    const bool ckpt_bf16 = p.flags & FLAG_CKPT_BF16;
    auto store_outputs = [&](int ph) {       // outputs of phase ph, published in buffer ph & 1
      const int c = nc - 1 - ph;
      const uint8_t* pub = smem + SM::PUB + (ph & 1) * SM::PUB_BYTES;
      const int tk = c * BT + 16 * hw + orow;   // dv2 tile hw
      const uint2 v = lds_tr8(pub + SM::PDV2 + hw * 512 + src);
      if (tk < sq.len) *reinterpret_cast<uint2*>(p.dv2 + ((row0 + tk) * p.HV + hv) * p.V + ocol) = v;
      if (p.dhc) {
#pragma unroll
        for (int md = hw; md < ND; md += 4) {
          const int64_t o = (((sq.cbase + c) * p.HV + hv) * K + 16 * md + orow) * p.V + ocol;
          const uint2 hi = lds_tr8(pub + SM::PDH + md * 512 + src);
          if (ckpt_bf16) {
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.dhc) + o) = hi;
          } else {
            const uint2 lo = lds_tr8(pub + SM::PDH + (ND + md) * 512 + src);
            *reinterpret_cast<uint4*>(static_cast<float*>(p.dhc) + o) =
                make_uint4((hi.x << 16) | (lo.x & 0xffffu), (hi.x & 0xffff0000u) | (lo.x >> 16),
                           (hi.y << 16) | (lo.y & 0xffffu), (hi.y & 0xffff0000u) | (lo.y >> 16));
          }
        }
      }
    };
    Ops ring[BWD_OUT_RING];
    {
      Ops first;
      load(0, first);
      stage(0, first);
    }
#pragma unroll
    for (int j = 0; j < PF; ++j) load(j + 1, ring[j]);
    barrier_lds();  // S0
    for (int t0 = 0; t0 < nphase; t0 += BWD_OUT_RING) {
#pragma unroll
      for (int j = 0; j < BWD_OUT_RING; ++j) {
        const int ph = t0 + j;
        // ring[j] holds the operands of phase ph + 1
        load(ph + 1 + PF, ring[(j + PF) % BWD_OUT_RING]);
        if (ph >= 1 && ph <= nc) store_outputs(ph - 1);
        stage(ph + 1, ring[j]);
        barrier_lds();
      }
    }
  } else {
    // ============================ loader waves ============================
    // Loader lw moves operand lw (kg, qg, w) of a chunk: piece i of this lane is
    // row 8 (i & 7) + (ln >> 3), columns 64 (i >> 3) + 8 (ln & 7) .. +7, so one load
    // instruction covers 8 rows x 128 contiguous bytes, whole cache lines (16 rows x
    // 64 bytes, half lines, measured 2.4 % slower).
    constexpr int NLD = BT * K / 8 / 64;     // 16-byte pieces per lane and chunk
    const int lw = wave - 5;
    const uint16_t* X = lw == 0 ? p.kg : (lw == 1 ? p.qg : p.w);
    const int off = lw * SM::KT_BYTES;
    if (nc == 0) {                          // empty sequence: only keep the barrier count
      for (int ph = 0; ph <= nphase; ++ph) barrier_lds();
      return;
    }
    const int lrow = ln >> 3, lcol = 8 * (ln & 7);
    const uint16_t* Xb = X + (row0 * p.HV + hv) * K + lcol;
    const int64_t rstride = (int64_t)p.HV * K;
    auto fetch = [&](int ph, u32x4* dst) {
      const int c = chunk_of(ph);
#pragma unroll
      for (int q = 0; q < 8; ++q) {          // the eight rows of this lane
        const uint16_t* a = Xb + (int64_t)min(c * BT + 8 * q + lrow, sq.len - 1) * rstride;
#pragma unroll
        for (int i = q; i < NLD; i += 8) dst[i] = *reinterpret_cast<const u32x4*>(a + 64 * (i >> 3));
      }
    };
    auto put = [&](int ph, const u32x4* src) {
      const int c = chunk_of(ph);
      uint8_t* dst = smem + (ph & 1) * SM::STAGE + off + (lrow * SM::RS + lcol) * 2;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool ok = c * BT + 8 * q + lrow < sq.len;
#pragma unroll
        for (int i = q; i < NLD; i += 8)
          *reinterpret_cast<u32x4*>(dst + (8 * q * SM::RS + 64 * (i >> 3)) * 2) = ok ? src[i] : u32x4{0, 0, 0, 0};
      }
    };
    u32x4 ra[NLD], rb[NLD], rc[NLD];
    fetch(0, ra);
    fetch(1, rb);
    fetch(2, rc);
    put(0, ra);
    barrier_lds();  // S0: phase 0 in LDS slot 0
    static_assert(BWD_LD_RING == 3, "the ring turn below is written out for three slots");
    for (int t0 = 0; t0 < nphase; t0 += BWD_LD_RING) {
      fetch(t0 + 3, ra);
      __builtin_amdgcn_sched_barrier(0);   // loads issue before the LDS writes
      put(t0 + 1, rb);
      barrier_lds();
      fetch(t0 + 4, rb);
      __builtin_amdgcn_sched_barrier(0);
      put(t0 + 2, rc);
      barrier_lds();
      fetch(t0 + 5, rc);
      __builtin_amdgcn_sched_barrier(0);
      put(t0 + 3, ra);
      barrier_lds();
    }
  }
}

hipError_t launch_bwd_dhu(const BwdParams& p, hipStream_t s) {
  const int64_t items = (int64_t)p.N * p.HV * (p.V / BV);
  if (items == 0) return hipSuccess;
  // longest-first order: whole rounds of eight units, V / 16 workgroups each
  const int grid = (int)(p.order ? ((int64_t)p.N * p.HV + 7) / 8 * 8 * (p.V / BV) : (items + 7) / 8 * 8);
  if (p.K == 128)
    hipLaunchKernelGGL((bwd_dhu_kernel<128>), dim3(grid), dim3(BWD_THREADS), 0, s, p, (int)items);
  else
    hipLaunchKernelGGL((bwd_dhu_kernel<64>), dim3(grid), dim3(BWD_THREADS), 0, s, p, (int)items);
  return hipGetLastError();
}

}  // namespace kda
