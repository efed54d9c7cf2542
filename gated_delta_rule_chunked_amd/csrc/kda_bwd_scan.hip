// kda_bwd_scan.hip -- segmented 64-column reverse state scan of the KDA chunked backward
// (gfx950).
//
// The recursion of kda_bwd.hip (the kernel-fun bwd_dhu module docstring), per chunk c of a
// sequence, newest first, with dh [K, V] fp32 starting at dht (or 0):
//   dhc[c] = dh;   dv2 = kg dh + dv;   dh <- diag(exp2 gd) dh + scale qg^T do - w^T dv2
// is affine in dh:  dh <- A_c dh + e_c  with  A_c = diag(exp2 gd) - w^T kg.  As the forward's
// segmented scan does (kda_scan.hip), a workgroup covers 64 value columns (four 16-column
// column waves that share one staged copy of the chunk's K-wide operands) of one segment of
// seg_L consecutive chunks, and segments are joined through their affine maps, here with time
// reversed (a segment hands its final dh to the next older one):
//   * the state pass computes, for every segment but a sequence's oldest, b (the dh the segment
//     hands on: from dht for the newest segment, from zero for the others) and, for every
//     segment but the newest and the oldest, M = A_first ... A_last (its chunks' transitions,
//     applied newest first), by scanning the columns of the identity with do = dv = 0.  A
//     column wave advances the b columns and the M columns of its group together, over one
//     staged copy of the operands (the loaders, not the products, bound a chunk);
//   * the full pass starts segment s (of S) from dh = dht for s = S-1, b_{S-1} for s = S-2 and
//     M_{s+1} dh_{s+1} + b_{s+1} below, and writes dv2, the checkpoints dhc and, after the
//     oldest segment, dh0.
// b is kept in fp32 and M in bf16, in the register orders of the forward's segment buffers
// (b in the column waves' C layout, M as the P-order A fragments of M dh).
//
// Eight waves per workgroup, one barrier per chunk:
//   waves 0-3 (column waves): wave c holds dh for columns 16c..16c+15 of the group in the C
//     layout of 16x16 MFMA tiles and runs a chunk's three products on bf16 MFMA: DV = kg dh onto
//     dv, QD = qg^T do and dh <- alpha dh + scale QD - w^T dv2 (the token contractions read
//     row-major LDS tiles through the transpose read).  In the full pass each column wave
//     stores its own outputs, the checkpoint and dv2, through its own corner of LDS: C-layout
//     tiles written, read back by the transpose read as row segments of 8 (bf16) or 16 (fp32)
//     bytes, no barrier needed since the corner is the wave's own.
//   waves 4-7 (loader waves): waves 4-6 one K-wide operand each (kg, qg, w), wave 7 the
//     group's do and dv rows and the chunk's decay row; a register ring three chunks deep,
//     copied into the free slot of a two-slot LDS ring.

#include "kda_device.hpp"
#include "kda_internal.hpp"

#include <algorithm>

namespace kda {

constexpr int BSCAN_THREADS = 512;
constexpr int BSCAN_RING = 3;   // chunks in flight per loader wave
enum BScanMode { BS_FULL = 0, BS_STATE = 1 };

template <int K, int MODE>
struct BScanSmem {
  // Row-major [64][K] tiles padded by 16 elements, as in kda_bwd.hip: eight consecutive rows
  // start on eight different groups of 8 banks, for both the row writes and the transpose reads.
  static constexpr int RS = K + 16;
  static constexpr int KT = BT * RS * 2;
  static constexpr int KG = 0, QG = KT, W = 2 * KT;
  static constexpr int VT = BT * BV * 2;            // one [64][16] bf16 tile
  static constexpr int DO = 3 * KT;                 // do: [4 column waves][64][16]
  static constexpr int DV = DO + 4 * VT;            // dv: [4 column waves][64][16]
  static constexpr int ALPHA = DV + 4 * VT;         // exp2(gd), fp32 [K]
  static constexpr int SLOT = ALPHA + K * 4;
  static constexpr int PUB = 2 * SLOT;              // full pass: each column wave's output corner
  static constexpr int PUB_WAVE = 4 * 512;          // four C-layout tiles [64 lanes][8 bytes]
  static constexpr int BYTES = PUB + (MODE == BS_FULL ? 4 * PUB_WAVE : 0);
  static_assert(BYTES <= 160 * 1024, "fits the LDS of one CU");
  static_assert(SLOT % 16 == 0 && (RS * 2) % 16 == 0, "16-byte aligned rows and slots");
};

// Phases of a segment of ncs chunks: whole ring turns, every role runs the same count.
__device__ __forceinline__ int bscan_phases(int ncs) {
  return (ncs + BSCAN_RING - 1) / BSCAN_RING * BSCAN_RING;
}

// ------------------------------------------------------------------ loader waves
// Loader lw (0..3) of a segment: 0-2 move kg, qg, w (a [64][K] tile each: lane ln takes rows
// 8 q + (ln >> 3), q = 0..7, and columns 64 (i >> 3) + 8 (ln & 7) .. +7 for its pieces i, so one
// load instruction covers 8 rows of 128 contiguous bytes); 3 moves the group's do and dv rows
// (lane ln: 16-byte column unit ln & 7 of the 64 columns, rows (ln >> 3) + 8 i) into one
// [64][16] tile per column wave, and the decay row exp2(g2) at the chunk's last valid row.
// Phase ph holds the ph-th chunk from the segment's newest; rows past the sequence are zero.
template <int K, int MODE>
__device__ __forceinline__ void bscan_loader(const BwdParams& p, uint8_t* smem, const SegLoc& sl, int hv, int grp,
                                             int lw, bool need_v) {
  using SM = BScanSmem<K, MODE>;
  constexpr int NLD = BT * K / 8 / 64;   // 16-byte pieces per lane of a [64][K] tile
  const int ln = threadIdx.x & 63;
  const int ncs = sl.ncs;
  if (ncs == 0) {
    barrier_lds();  // S0
    return;
  }
  const int nphase = bscan_phases(ncs);
  const int64_t row0 = (int64_t)sl.b * p.T + sl.bos;
  auto chunk_of = [&](int ph) { return sl.c0 + ncs - 1 - min(ph, ncs - 1); };   // the tail re-reads the oldest
  // qg is read only for b (the M columns have do = 0): without b columns its wave idles
  if (lw == 1 && !need_v) {
    for (int ph = 0; ph <= nphase; ++ph) barrier_lds();
    return;
  }
  if (lw < 3) {
    const uint16_t* X = lw == 0 ? p.kg : (lw == 1 ? p.qg : p.w);
    const int off = lw * SM::KT;
    const int lrow = ln >> 3, lcol = 8 * (ln & 7);
    const uint16_t* Xb = X + (row0 * p.HV + hv) * K + lcol;
    const int64_t rstride = (int64_t)p.HV * K;
    auto fetch = [&](int ph, u32x4* dst) {
      const int c = chunk_of(ph);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint16_t* a = Xb + (int64_t)min(c * BT + 8 * q + lrow, sl.len - 1) * rstride;
#pragma unroll
        for (int i = q; i < NLD; i += 8) dst[i] = *reinterpret_cast<const u32x4*>(a + 64 * (i >> 3));
      }
    };
    auto put = [&](int ph, const u32x4* src) {
      const int c = chunk_of(ph);
      uint8_t* dst = smem + (ph & 1) * SM::SLOT + off + (lrow * SM::RS + lcol) * 2;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool ok = c * BT + 8 * q + lrow < sl.len;
#pragma unroll
        for (int i = q; i < NLD; i += 8)
          *reinterpret_cast<u32x4*>(dst + (8 * q * SM::RS + 64 * (i >> 3)) * 2) = ok ? src[i] : u32x4{0, 0, 0, 0};
      }
    };
    u32x4 ring[BSCAN_RING][NLD];
#pragma unroll
    for (int j = 0; j < BSCAN_RING; ++j) fetch(j, ring[j]);
    put(0, ring[0]);
    barrier_lds();  // S0: the newest chunk in slot 0
    for (int t0 = 0; t0 < nphase; t0 += BSCAN_RING) {
#pragma unroll
      for (int j = 0; j < BSCAN_RING; ++j) {
        fetch(t0 + j + BSCAN_RING, ring[j]);
        __builtin_amdgcn_sched_barrier(0);   // loads issue before the LDS writes
        put(t0 + j + 1, ring[(j + 1) % BSCAN_RING]);
        barrier_lds();
      }
    }
    return;
  }
  // lw == 3: do and dv (only for b columns) and the decay row.  Every lane issues the same
  // loads whatever it keeps (no lane- or argument-dependent branches around loads, which
  // would leave the compiler's wait counting no choice but to wait for every load in flight).
  const int cu16 = ln & 7, vcw = cu16 >> 1, vhalf = cu16 & 1;
  const int vcol = min(grp * 64 + 8 * cu16, p.V - 8);        // columns past V: clamped, never used
  const bool alpha_lane = ln < K / 4;
  const int alane = min(ln, K / 4 - 1);
  const bool has_dv = p.dv != nullptr;
  const uint16_t* dvp = has_dv ? p.dv : p.dout;               // a valid address either way
  struct Ops {
    uint4 d[8], v[8];
    float4 g2;
  };
  auto fetch = [&](int ph, Ops& op) {
    const int c = chunk_of(ph);
    if (need_v) {   // uniform over the workgroup
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t t = row0 + min(c * BT + 8 * i + (ln >> 3), sl.len - 1);
        const int64_t vo = (t * p.HV + hv) * p.V + vcol;
        op.d[i] = *reinterpret_cast<const uint4*>(p.dout + vo);
        op.v[i] = *reinterpret_cast<const uint4*>(dvp + vo);
      }
    }
    const int64_t tl = row0 + min(c * BT + BT, sl.len) - 1;
    op.g2 = *reinterpret_cast<const float4*>(p.g2 + (tl * p.HV + hv) * K + 4 * alane);
  };
  auto put = [&](int ph, const Ops& op) {
    const int c = chunk_of(ph);
    uint8_t* st = smem + (ph & 1) * SM::SLOT;
    if (need_v) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 8 * i + (ln >> 3);
        const bool ok = c * BT + row < sl.len;
        const int o = (vcw * BT + row) * BV * 2 + vhalf * 16;
        *reinterpret_cast<uint4*>(st + SM::DO + o) = ok ? op.d[i] : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(st + SM::DV + o) = (ok && has_dv) ? op.v[i] : make_uint4(0, 0, 0, 0);
      }
    }
    if (alpha_lane)
      *reinterpret_cast<float4*>(st + SM::ALPHA + 16 * ln) =
          make_float4(__builtin_amdgcn_exp2f(op.g2.x), __builtin_amdgcn_exp2f(op.g2.y),
                      __builtin_amdgcn_exp2f(op.g2.z), __builtin_amdgcn_exp2f(op.g2.w));
  };
  Ops ring[BSCAN_RING];
#pragma unroll
  for (int j = 0; j < BSCAN_RING; ++j) fetch(j, ring[j]);
  put(0, ring[0]);
  barrier_lds();  // S0
  for (int t0 = 0; t0 < nphase; t0 += BSCAN_RING) {
#pragma unroll
    for (int j = 0; j < BSCAN_RING; ++j) {
      fetch(t0 + j + BSCAN_RING, ring[j]);
      __builtin_amdgcn_sched_barrier(0);
      put(t0 + j + 1, ring[(j + 1) % BSCAN_RING]);
      barrier_lds();
    }
  }
}

// ------------------------------------------------------------------ column waves
// Column wave cw of a segment.  The full pass advances dh for value columns
// 64 grp + 16 cw .. +15 and stores its outputs; the state pass advances, over the same
// staged operands, b for those value columns (do_b) and M for key columns 64 grp + 16 cw ..
// +15 (do_m).  A wave with neither keeps the barrier count only.
template <int K, int MODE>
__device__ __forceinline__ void bscan_column(const BwdParams& p, uint8_t* smem, const SegLoc& sl, int hv, int grp,
                                             int cw, bool do_b, bool do_m, int64_t sigma) {
  using SM = BScanSmem<K, MODE>;
  constexpr int S = K / 32, ND = K / 16;
  constexpr bool FULL = MODE == BS_FULL;
  const int ln = threadIdx.x & 63, r = ln & 15, g = ln >> 4;
  const int ncs = sl.ncs;
  const int nphase = ncs == 0 ? 0 : bscan_phases(ncs);
  if (!do_b && !do_m) {
    for (int ph = 0; ph <= nphase; ++ph) barrier_lds();
    return;
  }
  const bool state_bf16 = p.flags & FLAG_STATE_BF16;
  const int col = grp * 64 + BV * cw + r;                 // this lane's value (b, dh) or key (M) column
  const int64_t row0 = (int64_t)sl.b * p.T + sl.bos;
  // tile md: lane holds X[16 md + 4 g + rr][col], rr = 0..3
  f32x4 dh[ND], dm[ND];
  // b of segment sig in this wave's C-layout order: [segment][HV][V/16][K/16][64 lanes][4]
  auto b_at = [&](int64_t sig) {
    return reinterpret_cast<float4*>(p.bbuf) + ((sig * p.HV + hv) * (p.V / BV) + col / BV) * (int64_t)(ND * 64) + ln;
  };
  const bool newest = sl.s == sl.nseg - 1;
  if (do_m) {
#pragma unroll
    for (int md = 0; md < ND; ++md)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) dm[md][rr] = (16 * md + 4 * g + rr == col) ? 1.f : 0.f;
  }
  if (do_b) {
    if (newest) {
#pragma unroll
      for (int md = 0; md < ND; ++md)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d = 16 * md + 4 * g + rr;
          dh[md][rr] = p.dht ? load_state(state_bf16, p.dht, (((int64_t)sl.n * p.HV + hv) * K + d) * p.V + col) : 0.f;
        }
    } else if (!FULL) {
#pragma unroll
      for (int md = 0; md < ND; ++md) dh[md] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
      // full pass, an older segment: dh = b_{S-1}, then dh = M_{s'} dh + b_{s'} for the
      // segments s' between, newest first; a hop's loads are all issued before its products
      {
        const float4* bb = b_at(sl.sigma0 + sl.nseg - 1);
#pragma unroll
        for (int md = 0; md < ND; ++md) {
          const float4 t = bb[md * 64];
          dh[md] = f32x4{t.x, t.y, t.z, t.w};
        }
      }
      for (int s2 = sl.nseg - 2; s2 > sl.s; --s2) {
        f32x4 hn[ND];
        const float4* bb = b_at(sl.sigma0 + s2);
#pragma unroll
        for (int md = 0; md < ND; ++md) {
          const float4 t = bb[md * 64];
          hn[md] = f32x4{t.x, t.y, t.z, t.w};
        }
        const uint4* Mf = reinterpret_cast<const uint4*>(p.mbuf + ((sl.sigma0 + s2) * p.HV + hv) * (int64_t)K * K) + ln;
        uint4 mf[ND * S];
#pragma unroll
        for (int f = 0; f < ND * S; ++f) mf[f] = Mf[f * 64];
        uint2 hb[ND];
#pragma unroll
        for (int md = 0; md < ND; ++md) hb[md] = pack4(dh[md]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int md = 0; md < ND; ++md)
#pragma unroll
          for (int s3 = 0; s3 < S; ++s3)
            hn[md] = mfma16x32(as_frag(mf[md * S + s3]), cat(hb[2 * s3], hb[2 * s3 + 1]), hn[md]);
#pragma unroll
        for (int md = 0; md < ND; ++md) dh[md] = hn[md];
      }
    }
  }
  // per-lane parts of the LDS addresses (kda_bwd.hip's state wave)
  const int tb = ln >> 4, tj = (ln >> 2) & 3, ta = ln & 3;           // transpose-read source lane
  const int trK = ((4 * tb + tj) * SM::RS + 4 * ta) * 2;             // in a [64][K] tile
  const int tr16 = ((4 * tb + tj) * BV + 4 * ta) * 2;                // in a [64][16] tile
  const int kgA = (r * SM::RS + 4 * g) * 2;                          // A fragment of kg
  const bool ckpt_bf16 = p.flags & FLAG_CKPT_BF16;
  // this wave's output corner: four C-layout tiles; reading slot `src` of a tile with the
  // transpose read gives this lane row (ln & 15), columns 4 (ln >> 4) .. +3 of the tile (the
  // slot of C lane g = ln & 3, r = 4 (ln >> 4) + ((ln >> 2) & 3))
  uint8_t* corner = smem + SM::PUB + cw * SM::PUB_WAVE;
  const int src = (16 * (ln & 3) + 4 * (ln >> 4) + ((ln >> 2) & 3)) * 8;
  const int orow = ln & 15;
  const int64_t ocol = grp * 64 + BV * cw + 4 * (ln >> 4);
  barrier_lds();  // S0
  for (int ph = 0; ph < nphase; ++ph) {
    if (ph < ncs) {
      const int c = sl.c0 + ncs - 1 - ph;            // newest first
      const uint8_t* st = smem + (ph & 1) * SM::SLOT;
      uint2 hb[ND], hm[ND];
      if (do_b) {
#pragma unroll
        for (int md = 0; md < ND; ++md) hb[md] = pack4(dh[md]);
      }
      if (do_m) {
#pragma unroll
        for (int md = 0; md < ND; ++md) hm[md] = pack4(dm[md]);
      }
      if (FULL && p.dhc) {
        // the checkpoint (dh before this chunk's update) through the corner, four tiles at a
        // time: bf16 as the packed tiles, fp32 as a tile of the high and one of the low 16-bit
        // halves (rejoined after the read, exactly)
        const int64_t cbase = (((sl.cbase + c) * p.HV + hv) * K + orow) * (int64_t)p.V + ocol;
        if (ckpt_bf16) {
#pragma unroll
          for (int m4 = 0; m4 < ND; m4 += 4) {
#pragma unroll
            for (int q = 0; q < 4; ++q) *reinterpret_cast<uint2*>(corner + (q * 64 + ln) * 8) = hb[m4 + q];
            asm volatile("" ::: "memory");   // in-order LDS: the reads see this wave's writes
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint2 v = lds_tr8(corner + q * 512 + src);
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.dhc) + cbase + (int64_t)(16 * (m4 + q)) * p.V) = v;
            }
            asm volatile("" ::: "memory");
          }
        } else {
#pragma unroll
          for (int m2 = 0; m2 < ND; m2 += 2) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const f32x4 x = dh[m2 + q];
              const uint32_t u0 = f2u(x[0]), u1 = f2u(x[1]), u2 = f2u(x[2]), u3 = f2u(x[3]);
              *reinterpret_cast<uint2*>(corner + ((2 * q) * 64 + ln) * 8) =
                  make_uint2((u0 >> 16) | (u1 & 0xffff0000u), (u2 >> 16) | (u3 & 0xffff0000u));
              *reinterpret_cast<uint2*>(corner + ((2 * q + 1) * 64 + ln) * 8) =
                  make_uint2((u0 & 0xffffu) | (u1 << 16), (u2 & 0xffffu) | (u3 << 16));
            }
            asm volatile("" ::: "memory");
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const uint2 hi = lds_tr8(corner + (2 * q) * 512 + src);
              const uint2 lo = lds_tr8(corner + (2 * q + 1) * 512 + src);
              *reinterpret_cast<uint4*>(static_cast<float*>(p.dhc) + cbase + (int64_t)(16 * (m2 + q)) * p.V) =
                  make_uint4((hi.x << 16) | (lo.x & 0xffffu), (hi.x & 0xffff0000u) | (lo.x >> 16),
                             (hi.y << 16) | (lo.y & 0xffffu), (hi.y & 0xffff0000u) | (lo.y >> 16));
            }
            asm volatile("" ::: "memory");
          }
        }
      }
      // batch 1: kg A fragments, shared by the b and M columns
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
      // M: kg dm, negated in bf16 as the B operand of w^T (kg dm)
      uint2 vm[4] = {}, vp[4] = {};
      if (do_m) {
        f32x4 accm[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) accm[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const bf16x8 hms = cat(hm[2 * s], hm[2 * s + 1]);
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) accm[mb] = mfma16x32(cat(kl[mb * S + s], kh[mb * S + s]), hms, accm[mb]);
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          vm[mb] = pack4(accm[mb]);
          vm[mb].x ^= 0x80008000u;
          vm[mb].y ^= 0x80008000u;
        }
      }
      // b: dv2 = kg dh + dv in fp32, then bf16 (the full pass stores it through the corner,
      // as 8-byte row segments); negated, the B operand of w^T dv2
      if (do_b) {
        f32x4 acc[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const uint2 dvi = lds_tr8(st + SM::DV + cw * SM::VT + tr16 + mb * 16 * BV * 2);
          acc[mb] = f32x4{bflo(dvi.x), bfhi(dvi.x), bflo(dvi.y), bfhi(dvi.y)};
        }
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const bf16x8 hbs = cat(hb[2 * s], hb[2 * s + 1]);
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) acc[mb] = mfma16x32(cat(kl[mb * S + s], kh[mb * S + s]), hbs, acc[mb]);
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) vp[mb] = pack4(acc[mb]);
        if (FULL) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) *reinterpret_cast<uint2*>(corner + (mb * 64 + ln) * 8) = vp[mb];
          asm volatile("" ::: "memory");
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            const uint2 v = lds_tr8(corner + mb * 512 + src);
            const int tk = c * BT + 16 * mb + orow;
            if (tk < sl.len) *reinterpret_cast<uint2*>(p.dv2 + ((row0 + tk) * p.HV + hv) * p.V + ocol) = v;
          }
          asm volatile("" ::: "memory");
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          vp[mb].x ^= 0x80008000u;
          vp[mb].y ^= 0x80008000u;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // batch 2 (b only; the M columns have do = 0): QD = qg^T do, token contractions in P-order
      f32x4 qd[ND];
      if (do_b) {
        uint2 dol[2], doh[2], ql[2 * ND], qh[2 * ND];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          dol[s2] = lds_tr8(st + SM::DO + cw * SM::VT + tr16 + (32 * s2) * BV * 2);
          doh[s2] = lds_tr8(st + SM::DO + cw * SM::VT + tr16 + (32 * s2 + 16) * BV * 2);
        }
#pragma unroll
        for (int md = 0; md < ND; ++md)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const uint8_t* a = st + SM::QG + trK + ((32 * s2) * SM::RS + 16 * md) * 2;
            ql[md * 2 + s2] = lds_tr8(a);
            qh[md * 2 + s2] = lds_tr8(a + 16 * SM::RS * 2);
          }
#pragma unroll
        for (int md = 0; md < ND; ++md) {
          qd[md] = mfma16x32(cat(ql[md * 2], qh[md * 2]), cat(dol[0], doh[0]), f32x4{0.f, 0.f, 0.f, 0.f});
          qd[md] = mfma16x32(cat(ql[md * 2 + 1], qh[md * 2 + 1]), cat(dol[1], doh[1]), qd[md]);
        }
      }
      // batch 3, in two halves of the key rows: w^T A fragments and the decay (shared), then
      //   dh <- diag(alpha) dh + scale QD - w^T dv2;   dm <- diag(alpha) dm - w^T (kg dm)
      const bf16x8 vn0 = cat(vp[0], vp[1]), vn1 = cat(vp[2], vp[3]);
      const bf16x8 wn0 = cat(vm[0], vm[1]), wn1 = cat(vm[2], vm[3]);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        constexpr int NH = ND / 2;
        uint2 wl[2 * NH], wh[2 * NH];
        float4 al[NH];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NH; ++m) {
          const int md = h2 * NH + m;
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const uint8_t* a = st + SM::W + trK + ((32 * s2) * SM::RS + 16 * md) * 2;
            wl[m * 2 + s2] = lds_tr8(a);
            wh[m * 2 + s2] = lds_tr8(a + 16 * SM::RS * 2);
          }
          al[m] = *reinterpret_cast<const float4*>(st + SM::ALPHA + (16 * md + 4 * g) * 4);
        }
        if (do_b) {
#pragma unroll
          for (int m = 0; m < NH; ++m) {
            const int md = h2 * NH + m;
            f32x4 x;
            x[0] = al[m].x * dh[md][0] + p.scale * qd[md][0];
            x[1] = al[m].y * dh[md][1] + p.scale * qd[md][1];
            x[2] = al[m].z * dh[md][2] + p.scale * qd[md][2];
            x[3] = al[m].w * dh[md][3] + p.scale * qd[md][3];
            x = mfma16x32(cat(wl[m * 2], wh[m * 2]), vn0, x);
            dh[md] = mfma16x32(cat(wl[m * 2 + 1], wh[m * 2 + 1]), vn1, x);
          }
        }
        if (do_m) {
#pragma unroll
          for (int m = 0; m < NH; ++m) {
            const int md = h2 * NH + m;
            f32x4 x;
            x[0] = al[m].x * dm[md][0];
            x[1] = al[m].y * dm[md][1];
            x[2] = al[m].z * dm[md][2];
            x[3] = al[m].w * dm[md][3];
            x = mfma16x32(cat(wl[m * 2], wh[m * 2]), wn0, x);
            dm[md] = mfma16x32(cat(wl[m * 2 + 1], wh[m * 2 + 1]), wn1, x);
          }
        }
      }
    }
    barrier_lds();
  }
  // the segment's results
  if (!FULL && do_b) {
    float4* bb = b_at(sigma);
#pragma unroll
    for (int md = 0; md < ND; ++md) bb[md * 64] = make_float4(dh[md][0], dh[md][1], dh[md][2], dh[md][3]);
  }
  if (!FULL && do_m) {
    // M as P-order A fragments of the products M dh: fragment (md, s3) holds rows 16 md..,
    // columns 32 s3..; this lane's column col lands in lane group gp, element e, and its rows
    // 16 md + 4 g + rr in lanes 16 gp + 4 g + rr
    uint16_t* mm = p.mbuf + (sigma * p.HV + hv) * (int64_t)K * K;
    const int s3 = col >> 5, q = col & 31;
    const int gp = (q & 15) >> 2, e = (q & 3) + 4 * (q >> 4);
#pragma unroll
    for (int md = 0; md < ND; ++md)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) mm[((md * S + s3) * 64 + 16 * gp + 4 * g + rr) * 8 + e] = f2bf(dm[md][rr]);
  }
  if (FULL && p.dh0 && sl.s == 0) {
    int sv = p.V;
    asm volatile("" : "+s"(sv));   // opaque row stride: the row offsets are not kept live through the loop
#pragma unroll
    for (int md = 0; md < ND; ++md)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d = 16 * md + 4 * g + rr;
        store_state(state_bf16, p.dh0, (((int64_t)sl.n * p.HV + hv) * K + d) * (int64_t)sv + col, dh[md][rr]);
      }
  }
}

// State pass: item = (sigma * HV + hv) * NJ + j, NJ = max(V/64, K/64) rounded up: b for value
// columns 64 j.. (every segment but a sequence's oldest) and M for key columns 64 j.. (every
// segment but the newest and the oldest), in one workgroup over one set of staged operands.
template <int K>
__global__ __launch_bounds__(BSCAN_THREADS, 1) void bscan_state_kernel(BwdParams p, int n_items) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[BScanSmem<K, BS_STATE>::BYTES];
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  if (item >= n_items) return;
  if (p.cu != nullptr && p.table[p.N + 1] != 0) return;   // rejected cu_seqlens: the full pass reports it
  const int NCG = (p.V + 63) / 64, NJ = max(NCG, K / 64);
  const int j = item % NJ;
  const int hv = (item / NJ) % p.HV;
  const int64_t sigma = item / (NJ * p.HV);
  SegLoc sl;
  if (!locate_segment(p, sigma, sl)) return;
  const int nb = (sl.s > 0 && j < NCG) ? min(4, (p.V - 64 * j) / BV) : 0;
  const int nm = (sl.s > 0 && sl.s < sl.nseg - 1 && j < K / 64) ? 4 : 0;
  if (nb == 0 && nm == 0) return;                            // uniform over the workgroup
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave >= 4) bscan_loader<K, BS_STATE>(p, smem, sl, hv, j, wave - 4, nb > 0);
  else bscan_column<K, BS_STATE>(p, smem, sl, hv, j, wave, wave < nb, wave < nm, sigma);
}

// Full pass: item = (sigma * HV + hv) * NCG + cg.
template <int K>
__global__ __launch_bounds__(BSCAN_THREADS, 1) void bscan_full_kernel(BwdParams p, int n_items) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[BScanSmem<K, BS_FULL>::BYTES];
  const int item = p.order ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
  if (p.order) n_items = (int)gridDim.x;
  if (item >= n_items) return;
  const int tid = threadIdx.x;
  if (p.cu != nullptr && p.table[p.N + 1] != 0) {
    // rejected cu_seqlens: poison all of dv2 and dh0, grid-strided
    const int64_t total = (int64_t)p.B * p.T * p.HV * p.V;
    for (int64_t idx = (int64_t)item * BSCAN_THREADS + tid; idx < total; idx += (int64_t)n_items * BSCAN_THREADS)
      p.dv2[idx] = 0x7fc0;
    if (p.dh0) {
      const int64_t nh = (int64_t)p.N * p.HV * K * p.V;
      for (int64_t idx = (int64_t)item * BSCAN_THREADS + tid; idx < nh; idx += (int64_t)n_items * BSCAN_THREADS)
        store_state(p.flags & FLAG_STATE_BF16, p.dh0, idx, __builtin_nanf(""));
    }
    return;
  }
  const int NCG = (p.V + 63) / 64;
  int cg, hv;
  int64_t sigma;
  if (p.order) {
    // varlen, one segment per sequence: (sequence rank, head) units in dispatch order, the
    // longest sequences first; a unit's column groups follow in consecutive rounds of eight
    const int b = blockIdx.x, rnd = b >> 3;
    const int64_t u = (int64_t)(rnd / NCG) * 8 + (b & 7);
    if (u >= (int64_t)p.N * p.HV) return;
    cg = rnd % NCG;
    hv = (int)(u % p.HV);
    sigma = p.order[u / p.HV];
    if ((uint64_t)sigma >= (uint64_t)p.N) return;   // never for an order the chunk table wrote
  } else {
    cg = item % NCG;
    hv = (item / NCG) % p.HV;
    sigma = item / (NCG * p.HV);
  }
  SegLoc sl;
  if (!locate_segment(p, sigma, sl)) return;
  const int ntiles = min(4, (p.V - 64 * cg) / BV);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave >= 4) bscan_loader<K, BS_FULL>(p, smem, sl, hv, cg, wave - 4, true);
  else bscan_column<K, BS_FULL>(p, smem, sl, hv, cg, wave, wave < ntiles, false, sigma);
}

template <int K>
static hipError_t launch_bwd_scan_k(const BwdParams& p, hipStream_t s) {
  const int64_t NCG = (p.V + 63) / 64;
  if (p.bbuf != nullptr) {
    const int64_t items = p.max_segs * p.HV * std::max<int64_t>(NCG, K / 64);
    hipLaunchKernelGGL((bscan_state_kernel<K>), dim3((int)((items + 7) / 8 * 8)), dim3(BSCAN_THREADS), 0, s, p,
                       (int)items);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t items = p.max_segs * p.HV * NCG;
  const int64_t grid = p.order ? ((int64_t)p.N * p.HV + 7) / 8 * 8 * NCG : (items + 7) / 8 * 8;
  hipLaunchKernelGGL((bscan_full_kernel<K>), dim3((int)grid), dim3(BSCAN_THREADS), 0, s, p, (int)items);
  return hipGetLastError();
}

hipError_t launch_bwd_scan(const BwdParams& p, hipStream_t s) {
  if (p.max_segs * p.HV == 0) return hipSuccess;
  return p.K == 128 ? launch_bwd_scan_k<128>(p, s) : launch_bwd_scan_k<64>(p, s);
}

}  // namespace kda
