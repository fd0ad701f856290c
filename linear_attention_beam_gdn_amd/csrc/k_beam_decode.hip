// Fused shared-context decode step for beams that share one state per
// request (OneLA §3.4, Figure 5; replay equations of §3.2; ancestry of §3.3).
//
// Work split.  One workgroup takes one (request r, head h), a slice of VS
// value rows (all of d_v up to 128; wider d_v is cut into slices, since every
// value row's replay is independent given the per-beam dot products, which
// each slice forms itself) and a chunk of beams.  Its NW waves split the slice (RPW value rows each, the B_V tile
// of §3.4) and each wave keeps its part of the shared state S0[r,h] in
// registers for the whole beam chunk, in the A-operand layout of the gfx950
// bf16 MFMA (16x16x32): S0 is read from memory once per workgroup and reused
// by every beam of the chunk.  FP32 S0 is split on chip into NPL bf16 planes
// (hi + mid + lo); q and k arrive as bf16, so each plane product is exact and
// the MFMA accumulates the projections S0^T q and S0^T k in FP32.
//
// Beams are processed 16 at a time (the MFMA N dimension).  Lane (g, c) of a
// wave (g = lane / 16, c = lane % 16) owns beam c of the tile: it holds a
// quarter of that beam's q and k (the B operand) and, after the MFMA, 4*MT
// consecutive value rows of its projections (the C layout).  The dot products
// k_j . q and k_j . k of the replay are reduced over the four lane groups of
// the beam; the value-side updates are per lane, so the replay never leaves
// registers.
#include "beam_common.h"

namespace gdn {
namespace {

template <int DK, int DV, bool CH = false>
struct BeamGeom {
  static_assert(DK == 16 || DK == 32 || DK % 64 == 0, "d_k must be 16, 32 or a multiple of 64");
  static_assert(DV % 16 == 0, "d_v must be a multiple of 16");
  // value rows per wave: 16 for d_k > 128, so that a wave's state slice (three
  // planes of d_k / 32 MFMA steps) stays within its registers
  static constexpr int RPW = (DK <= 128 && DV % 32 == 0) ? 32 : 16;
  // value rows per workgroup: wider d_v is split over NVS workgroups.  Up to
  // eight waves (two per SIMD, 256 registers each); four (one per SIMD, with
  // the whole register file) for d_k = 256 and for channel decay, whose
  // lanes also hold their key channels' decays and probe weights
  static constexpr int VS0 = DK > 128 ? 64 : (CH ? 128 : 256);
  static constexpr int VS = DV < VS0 ? DV : VS0;
  static_assert(DV % VS == 0, "d_v must split evenly over value slices");
  static constexpr int NVS = DV / VS;                   // value slices
  static constexpr int NW = VS / RPW;                   // waves per workgroup
  static constexpr int MT = RPW / 16;                   // 16-row MFMA tiles per wave
  static constexpr int KS = (DK + 31) / 32;             // 32-deep MFMA steps over d_k
  static constexpr int VPL = 4 * MT;                    // value rows per lane
};

template <int DK, int DV, bool CH, int NPL>
__global__ __launch_bounds__((BeamGeom<DK, DV, CH>::NW * 64)) void k_beam_decode(BeamArgs a) {
  using G = BeamGeom<DK, DV, CH>;
  constexpr int A = CH ? DK : 1;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int c = lane & 15;

  // Workgroups are handed to the 8 XCDs round-robin; renumber them so that
  // the chunks of one (r, h) run on the same XCD and share its L2.
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int chunk_id = bid % a.nchunk;
  const int vsl = (bid / a.nchunk) % G::NVS;
  const int rh = bid / (a.nchunk * G::NVS);
  const int h = rh % a.H;
  const int r = rh / a.H;
  const int b_begin = chunk_id * a.chunk;
  const int b_end = min(b_begin + a.chunk, a.Wt);
  const int t = a.t;
  const int vs0 = vsl * G::VS;                    // first value row of the slice
  const int dv0 = vs0 + w * G::RPW + g * G::VPL;  // first value row held by this lane

  // ---- this wave's slice of S0[r, h] as bf16 planes in MFMA A layout.
  // A row m of tile mt is value row vs0 + w*RPW + (m/4)*VPL + mt*4 + m%4, so that
  // C row 4g+i of tile mt lands on value row dv0 + mt*4 + i.
  u32x4 As[G::MT][G::KS][NPL];
  {
    const float* S = a.S + ((size_t)r * a.H + h) * DK * DV;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) {
      const int col = vs0 + w * G::RPW + (c >> 2) * G::VPL + mt * 4 + (c & 3);
#pragma unroll
      for (int s = 0; s < G::KS; ++s) {
        const int k0 = kchunk<DK>(g, s);
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = klive<DK>(g) ? S[(size_t)(k0 + e) * DV + col] : 0.f;
        split_planes<NPL>(x, As[mt][s]);
      }
    }
  }

  // the first value slice writes what is not per value row: ancestry, the
  // record key (once per key head) and the record decay
  const bool slice_writer = vsl == 0;
  const bool anc_writer = (h == 0) && slice_writer && (w == 0) && (g == 0);
  const int hk = h / a.gq;
  const bool key_writer = h % a.gq == 0;

  for (int b0 = b_begin; b0 < b_end; b0 += 16) {
    const int b = b0 + c;
    const bool valid = b < b_end;
    const size_t tok = ((size_t)r * a.Wt + (valid ? b : 0)) * a.H + h;
    const size_t rec_t = (((size_t)t * a.R + r) * a.Wm + (valid ? b : 0)) * a.H + h;
    // the key head's q and k, and its record key (one writer per key head)
    const size_t tok_k = ((size_t)r * a.Wt + (valid ? b : 0)) * a.Hk + hk;
    const size_t rec_tk = (((size_t)t * a.R + r) * a.Wm + (valid ? b : 0)) * a.Hk + hk;

    // ---- ancestry (§3.3): parent slot and the parent's own ancestry row
    int par = 0;
    if (t > 0 && valid) {
      const int raw = a.parent[(size_t)r * a.Wt + b];
      if (anc_writer) check_parent(a, raw);
      par = clampi(raw, 0, a.Wm - 1);
    }
    const int32_t* prow = a.anc + (((size_t)(t > 0 ? t - 1 : 0) * a.R + r) * a.Wm + par) * a.L;
    // Record slots: with scalar decay a step's records sit at the beams'
    // order keys (the last entry of their ancestry rows: this kernel takes
    // beams in index order, so its key is the index; the fused kernel's is
    // the beam's depth-first position), so the parent's slot is the key in
    // its row; at step 0 and with channel decay a slot is the beam index.
    auto slot_at = [&](int j) -> int {
      if (!valid) return 0;
      if (j == t - 1) return (!CH && t >= 2) ? clampi(prow[a.L - 1], 0, a.Wm - 1) : par;
      return clampi(prow[j], 0, a.Wm - 1);
    };
    if (anc_writer && valid) a.anc[(((size_t)t * a.R + r) * a.Wm + b) * a.L + a.L - 1] = b;  // this step's key
    auto rec_at = [&](int j, int slot) -> size_t {
      return (((size_t)j * a.R + r) * a.Wm + slot) * a.H + h;
    };
    auto rec_at_k = [&](int j, int slot) -> size_t {
      return (((size_t)j * a.R + r) * a.Wm + slot) * a.Hk + hk;
    };

    // ---- current q and k (B operand chunks)
    u32x4 qf[G::KS], kf[G::KS];
#pragma unroll
    for (int s = 0; s < G::KS; ++s) {
      const int k0 = kchunk<DK>(g, s);
      const bool ld = valid && klive<DK>(g);
      qf[s] = ld ? *reinterpret_cast<const u32x4*>(a.q + tok_k * DK + k0) : u32x4{0, 0, 0, 0};
      kf[s] = ld ? *reinterpret_cast<const u32x4*>(a.k + tok_k * DK + k0) : u32x4{0, 0, 0, 0};
    }

    // current decay: scalar, or this lane's key channels of the vector
    float at = 0.f;
    float acur[CH ? G::KS * 8 : 1];
    if constexpr (!CH) {
      at = valid ? a.alpha[tok] : 0.f;
    } else {
#pragma unroll
      for (int s = 0; s < G::KS; ++s) {
        if (valid && klive<DK>(g)) load_f32x8(a.alpha + tok * DK + kchunk<DK>(g, s), acur + 8 * s);
        else
#pragma unroll
          for (int e = 0; e < 8; ++e) acur[8 * s + e] = 0.f;
      }
    }

    // ---- S0^T [q | k] on the matrix cores
    f32x4 uq[G::MT], uk[G::MT];
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) {
      uq[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      uk[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (!CH) {
#pragma unroll
      for (int s = 0; s < G::KS; ++s)
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
          for (int p = NPL - 1; p >= 0; --p) {
            uq[mt] = mfma16x16x32(As[mt][s][p], qf[s], uq[mt]);
            uk[mt] = mfma16x16x32(As[mt][s][p], kf[s], uk[mt]);
          }
    } else {
      // Channel decay: the probes are (prod_{i<=t} a_i) * x over the beam's
      // chain (FP32), split into two bf16 planes; plane pairs whose combined
      // weight is below 2^-16 relative are dropped.
      float cum[G::KS * 8];
#pragma unroll
      for (int i = 0; i < G::KS * 8; ++i) cum[i] = acur[i];
      for (int j = 0; j < t; ++j) {
        const size_t rj = rec_at(j, slot_at(j));
#pragma unroll
        for (int s = 0; s < G::KS; ++s) {
          float aj[8];
          if (valid && klive<DK>(g)) load_f32x8(a.rec_alpha + rj * A + kchunk<DK>(g, s), aj);
          else
#pragma unroll
            for (int e = 0; e < 8; ++e) aj[e] = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) cum[8 * s + e] *= aj[e];
        }
      }
#pragma unroll
      for (int s = 0; s < G::KS; ++s) {
        float xq[8], xk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xq[e] = cum[8 * s + e] * bf16x8_elem(qf[s], e);
          xk[e] = cum[8 * s + e] * bf16x8_elem(kf[s], e);
        }
        u32x4 pq[2], pk[2];
        split_planes<2>(xq, pq);
        split_planes<2>(xk, pk);
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) {
#pragma unroll
          for (int pa = NPL - 1; pa >= 0; --pa)
#pragma unroll
            for (int pb = 1; pb >= 0; --pb) {
              if (pa + pb >= NPL) continue;
              uq[mt] = mfma16x16x32(As[mt][s][pa], pq[pb], uq[mt]);
              uk[mt] = mfma16x16x32(As[mt][s][pa], pk[pb], uk[mt]);
            }
        }
      }
    }

    // k_t . q_t
    float sqq = 0.f;
#pragma unroll
    for (int s = 0; s < G::KS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) sqq += bf16x8_elem(kf[s], e) * bf16x8_elem(qf[s], e);
    sqq = sum_lane_groups(sqq);

    // ---- replay of the ancestral records (§3.2), gathered through h_t
    if constexpr (!CH) {
      for (int j = 0; j < t; ++j) {
        const int slot = slot_at(j);
        if (anc_writer && valid) a.anc[(((size_t)t * a.R + r) * a.Wm + b) * a.L + j] = slot;
        const size_t rj = rec_at(j, slot);
        float pq = 0.f, pk = 0.f;
#pragma unroll
        for (int s = 0; s < G::KS; ++s) {
          const bool ld = valid && klive<DK>(g);
          const u32x4 kj = ld ? *reinterpret_cast<const u32x4*>(a.rec_k + rec_at_k(j, slot) * DK + kchunk<DK>(g, s))
                              : u32x4{0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float kje = bf16x8_elem(kj, e);
            pq += kje * bf16x8_elem(qf[s], e);
            pk += kje * bf16x8_elem(kf[s], e);
          }
        }
        pq = sum_lane_groups(pq);
        pk = sum_lane_groups(pk);
        const float aj = valid ? a.rec_alpha[rj] : 0.f;
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) {
          const f32x4 dj = valid ? *reinterpret_cast<const f32x4*>(a.rec_delta + rj * DV + dv0 + mt * 4)
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uq[mt][i] = aj * uq[mt][i] + dj[i] * pq;
            uk[mt][i] = aj * uk[mt][i] + dj[i] * pk;
          }
        }
      }
    } else {
      // S_j^T y = S_{j-1}^T (a_j * y) + delta_j (k_j . y), from j = t-1 down;
      // P holds prod_{i=j+1..t} a_i on this lane's key channels.
      float P[G::KS * 8];
#pragma unroll
      for (int i = 0; i < G::KS * 8; ++i) P[i] = acur[i];
      for (int j = t - 1; j >= 0; --j) {
        const int slot = slot_at(j);
        if (anc_writer && valid) a.anc[(((size_t)t * a.R + r) * a.Wm + b) * a.L + j] = slot;
        const size_t rj = rec_at(j, slot);
        float pq = 0.f, pk = 0.f;
#pragma unroll
        for (int s = 0; s < G::KS; ++s) {
          const bool ld = valid && klive<DK>(g);
          const u32x4 kj = ld ? *reinterpret_cast<const u32x4*>(a.rec_k + rec_at_k(j, slot) * DK + kchunk<DK>(g, s))
                              : u32x4{0, 0, 0, 0};
          float aj[8];
          if (ld) load_f32x8(a.rec_alpha + rj * A + kchunk<DK>(g, s), aj);
          else
#pragma unroll
            for (int e = 0; e < 8; ++e) aj[e] = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float y = bf16x8_elem(kj, e) * P[8 * s + e];
            pq += y * bf16x8_elem(qf[s], e);
            pk += y * bf16x8_elem(kf[s], e);
            P[8 * s + e] *= aj[e];
          }
        }
        pq = sum_lane_groups(pq);
        pk = sum_lane_groups(pk);
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) {
          const f32x4 dj = valid ? *reinterpret_cast<const f32x4*>(a.rec_delta + rj * DV + dv0 + mt * 4)
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uq[mt][i] += dj[i] * pq;
            uk[mt][i] += dj[i] * pk;
          }
        }
      }
    }

    // ---- current transition and append (§3.2, §3.4)
    if (valid) {
      const float bt = a.beta[tok];
      float vv[G::VPL];
      if constexpr (G::VPL == 8) {
        const u32x4 vw = *reinterpret_cast<const u32x4*>(a.v + tok * DV + dv0);
#pragma unroll
        for (int i = 0; i < 8; ++i) vv[i] = bf16x8_elem(vw, i);
      } else {
        const u32x2 vw = *reinterpret_cast<const u32x2*>(a.v + tok * DV + dv0);
#pragma unroll
        for (int i = 0; i < 4; ++i) vv[i] = (i & 1) ? bf16_hi(vw[i >> 1]) : bf16_lo(vw[i >> 1]);
      }
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) {
        f32x4 d, out;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (!CH) {
            d[i] = bt * (vv[mt * 4 + i] - at * uk[mt][i]);
            out[i] = at * uq[mt][i] + d[i] * sqq;
          } else {
            d[i] = bt * (vv[mt * 4 + i] - uk[mt][i]);
            out[i] = uq[mt][i] + d[i] * sqq;
          }
        }
        *reinterpret_cast<f32x4*>(a.o + tok * DV + dv0 + mt * 4) = out;
        *reinterpret_cast<f32x4*>(a.rec_delta + rec_t * DV + dv0 + mt * 4) = d;
      }
      if (slice_writer && w == 0 && klive<DK>(g)) {
#pragma unroll
        for (int s = 0; s < G::KS; ++s) {
          const int k0 = kchunk<DK>(g, s);
          if (key_writer) *reinterpret_cast<u32x4*>(a.rec_k + rec_tk * DK + k0) = kf[s];
          if constexpr (CH) {
            *reinterpret_cast<f32x4*>(a.rec_alpha + rec_t * A + k0) =
                f32x4{acur[8 * s], acur[8 * s + 1], acur[8 * s + 2], acur[8 * s + 3]};
            *reinterpret_cast<f32x4*>(a.rec_alpha + rec_t * A + k0 + 4) =
                f32x4{acur[8 * s + 4], acur[8 * s + 5], acur[8 * s + 6], acur[8 * s + 7]};
          }
        }
        if constexpr (!CH)
          if (g == 0) a.rec_alpha[rec_t] = at;
      }
    }
  }
}

template <int DK, int DV, bool CH>
int launch(const gdn_shape& sh, const gdn_store& st, int t, int Wt, const StepIO& io,
           hipStream_t stream) {
  constexpr int NPL = CH ? 2 : 3;
  BeamArgs a;
  a.S = st.S;
  a.rec_delta = st.rec_delta;
  a.rec_k = st.rec_k;
  a.rec_alpha = st.rec_alpha;
  a.anc = st.anc;
  a.parent = io.parent;
  a.bad_parents = io.bad_parents;
  a.q = io.q;
  a.k = io.k;
  a.v = io.v;
  a.alpha = io.alpha;
  a.beta = io.beta;
  a.o = io.o;
  a.R = sh.R;
  a.Wm = sh.W_max;
  a.H = sh.H;
  a.L = sh.L_max;
  a.t = t;
  a.Wt = Wt;
  a.Hk = key_heads(sh);
  a.gq = sh.H / a.Hk;
  constexpr int NVS = BeamGeom<DK, DV, CH>::NVS;
  a.chunk = pick_chunk(sh.R * sh.H * NVS, Wt, 1 << 30, 2048);
  a.nchunk = (Wt + a.chunk - 1) / a.chunk;
  const long grid = (long)sh.R * sh.H * NVS * a.nchunk;
  if (grid > 0x7FFFFFFFL) return GDN_EINVAL;
  GDN_DISPATCH(io.ev_start, io.ev_stop, (k_beam_decode<DK, DV, CH, NPL>), dim3((unsigned)grid),
               dim3(BeamGeom<DK, DV, CH>::NW * 64), 0, stream, a);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_EHIP;
}

}  // namespace

int launch_beam_decode(const gdn_shape& sh, const gdn_store& st, int t, int Wt, const StepIO& io,
                       hipStream_t stream) {
  // GDN_BEAM_GENERIC=1 forces the register-only kernel (for A/B comparisons)
  const char* generic = getenv("GDN_BEAM_GENERIC");
  const bool force_generic = generic != nullptr && generic[0] == '1';
  if (beam_fused_supported(sh, t) && !force_generic) return launch_beam_fused(sh, st, t, Wt, io, stream);
  if (beam_fused_kda_supported(sh, t) && !force_generic) return launch_beam_fused_kda(sh, st, t, Wt, io, stream);
  const bool ch = sh.decay_kind == GDN_DECAY_CHANNEL;
#define GDN_CASE(DK_, DV_)                                                       \
  if (sh.dk == DK_ && sh.dv == DV_)                                              \
    return ch ? launch<DK_, DV_, true>(sh, st, t, Wt, io, stream)                \
              : launch<DK_, DV_, false>(sh, st, t, Wt, io, stream);
  GDN_CASE(16, 16)
  GDN_CASE(32, 32)
  GDN_CASE(64, 64)
  GDN_CASE(128, 128)
  GDN_CASE(128, 256)
  GDN_CASE(128, 512)
#undef GDN_CASE
  // d_k = 256: the scalar rule only (channel decay would hold d_k decays and
  // probe weights per lane on top of the state slice)
  if (!ch && sh.dk == 256) {
    if (sh.dv == 128) return launch<256, 128, false>(sh, st, t, Wt, io, stream);
    if (sh.dv == 256) return launch<256, 256, false>(sh, st, t, Wt, io, stream);
    if (sh.dv == 512) return launch<256, 512, false>(sh, st, t, Wt, io, stream);
  }
  return GDN_EUNSUPPORTED;
}

}  // namespace gdn
