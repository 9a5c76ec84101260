// Decode path of the double-binary layer: both sign-accumulate products of
// LoRDBA section 2 ("Kernel de Inferencia") / DBF section 2 ("Inferencia")
// over the packed bits with 16-entry signed subset-sum tables (dbf_lut.h),
// in one launch.
//
// Workgroups [0, n1) are stage 1 (rows of B2 against gamma . x, split along
// M into ks partials of w = beta . t in the workspace).  Workgroups
// [n1, n1 + n2) are stage 2 (rows of B1 against the summed w, times alpha,
// summed over the terms, y written once).  A stage-2 workgroup issues the
// loads of its first B1 bits, then waits until all stage-1 workgroups have
// published, so the B1 traffic overlaps stage 1.  Stage-2 workgroups have
// higher block indices than every stage-1 workgroup, so on each XCD every
// stage-1 workgroup is dispatched before a stage-2 workgroup can wait on it;
// the wait is bounded, and the last stage-2 workgroup to pass it resets the
// counters for the next call (or graph replay).
#include <type_traits>

#include "dbf_lut.h"

namespace dbf {
namespace {

using namespace lut;

struct Stage2 {
  TermPtrs t;
  int64_t T, N, R, nkb;
  int ks;
  const void* ws;
  int64_t rs;
  void* y;
  int y_dtype;
  int64_t ldy;
  int accumulate;
  int32_t* s2_out;
  int32_t* s1_out;  // int8 variant: exact S1, written by stage-2 workgroups of row tile 0
  Sync sync;        // n_prod = stage-1 workgroups, n_cons = stage-2 workgroups
  unsigned n2;
  int64_t nrt;      // row tiles of N; workgroup = (token block, row tile)
};

// The sum over the K-split partials of w_term[tok][k .. k + 4) (loads issued
// BATCH splits at a time, to bound the registers they hold; summed in split
// order), as stage 2's act4.
template <typename A, int MODE, int BATCH = 4>
__device__ __forceinline__ void w4(const Stage2& p, int term, int64_t tt, int64_t k, int64_t rt,
                                   A* v) {
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = A(0);
  if (tt >= p.T || k >= p.R) return;
  const int64_t base = (static_cast<int64_t>(term) * p.ks * p.T + tt) * p.rs + k;
  using PT = typename std::conditional<MODE == MODE_F, float, int32_t>::type;
  using PT4 = typename std::conditional<MODE == MODE_F, float4, int4>::type;
  const PT* wsp = static_cast<const PT*>(p.ws);
  // at most BATCH splits' loads in flight (registers); more splits take
  // further rounds
  constexpr int kBatch = BATCH;
  PT4 sum;
  {
    PT4 q[kBatch];
#pragma unroll
    for (int s = 0; s < kBatch; ++s)
      if (s < p.ks) q[s] = load_shared4<PT4>(wsp + base + s * p.T * p.rs);
    sum = q[0];
#pragma unroll
    for (int s = 1; s < kBatch; ++s)
      if (s < p.ks) {
        sum.x += q[s].x; sum.y += q[s].y; sum.z += q[s].z; sum.w += q[s].w;
      }
  }
#pragma unroll
  for (int s0 = kBatch; s0 < kMaxKS; s0 += kBatch) {
    if (s0 >= p.ks) break;
    PT4 q[kBatch];
#pragma unroll
    for (int s = 0; s < kBatch; ++s)
      if (s0 + s < p.ks) q[s] = load_shared4<PT4>(wsp + base + (s0 + s) * p.T * p.rs);
#pragma unroll
    for (int s = 0; s < kBatch; ++s)
      if (s0 + s < p.ks) {
        sum.x += q[s].x; sum.y += q[s].y; sum.z += q[s].z; sum.w += q[s].w;
      }
  }
  const PT sv[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (k + j >= p.R) continue;
    if constexpr (MODE == MODE_I8_BETA)
      v[j] = f16_bits_to_f32(p.t.beta[term][k + j]) * static_cast<float>(sv[j]);
    else
      v[j] = sv[j];
    if constexpr (MODE != MODE_F) {
      if (rt == 0 && p.s1_out) p.s1_out[(term * p.T + tt) * p.R + k + j] = sv[j];
    }
  }
}

template <typename A, int TB, int KW, int MODE, int NW>
__device__ __forceinline__ void stage2_role(const Stage2& p, int64_t bid2, A* tbl, A* red) {
  constexpr int PW = pw_of(TB);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t tblk = bid2 / p.nrt;
  const int64_t rt = bid2 - tblk * p.nrt;
  const int64_t row = rt * 64 + lane;
  constexpr int E = ents_per_thread<TB, KW, NW>();
  constexpr int64_t step = NW * PW;
  // alpha of this lane's row for every term, two to a register (inputs:
  // read before the wait, which waits for them anyway, by every lane with
  // the row clamped; none means 1)
  const int64_t arow = row < p.N ? row : p.N - 1;
  uint32_t aln[DBF_MAX_TERMS / 2];
#pragma unroll
  for (int q = 0; q < DBF_MAX_TERMS; q += 2) {
    const uint32_t lo = q < p.t.n && p.t.alpha[q] ? p.t.alpha[q][arow] : 0x3C00u;
    const uint32_t hi = q + 1 < p.t.n && p.t.alpha[q + 1] ? p.t.alpha[q + 1][arow] : 0x3C00u;
    aln[q / 2] = lo | (hi << 16);
  }
  uint32_t wd[PW][KW], wdn[PW][KW];
  load_pass_bits<TB, KW, NW>(p.t.b1[0], rt, p.nkb, 0, p.nkb, wd);
  wait_producers(p.sync, false);  // partials via load_shared4
  unsigned ticket = 0;
  {
    const int64_t tok0 = tblk * TB;
    float yacc[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) yacc[i] = 0.f;
    for (int term = 0; term < p.t.n; ++term) {
      A acc[TB];
#pragma unroll
      for (int i = 0; i < TB; ++i) acc[i] = A(0);
      for (int64_t kp = 0; kp < p.nkb; kp += step) {
        const int64_t kb_end = min(p.nkb, kp + step);
        const int ng = static_cast<int>((kb_end - kp) * 8 * KW);
        const int64_t kbase = kp * 32 * KW;
        // group g of the pass: w[tok][k .. k + 4) of this term
        auto act4 = [&](int tok, int g, A* v) { w4<A, MODE>(p, term, tok0 + tok, kbase + 4 * g, rt, v); };
        A v[E][4];
        load_acts<A, TB, KW, NW>(act4, ng, v);
        // issued after the partials, so their round trips overlap the tables
        // and lookups: the ticket and the next pass's signs (this term's next
        // K-blocks or the next term's first)
        if (kp == 0 && term == 0) ticket = take_ticket(p.sync);
        const bool more = kp + step < p.nkb, next_term = !more && term + 1 < p.t.n;
        if (more || next_term)  // one call: the two cases load the same registers
          load_pass_bits<TB, KW, NW>(p.t.b1[more ? term : term + 1], rt, p.nkb, more ? kp + step : 0,
                                 p.nkb, wdn);
        tables_and_lookups_v<A, TB, KW, NW>(v, tbl, ng, kp, kb_end, wd, acc);
        if (more || next_term) {
#pragma unroll
          for (int j = 0; j < PW; ++j)
#pragma unroll
            for (int w = 0; w < KW; ++w) wd[j][w] = wdn[j][w];
        }
      }
      reduce_waves<A, TB, NW>(red, acc);
      if (wv == 0 && row < p.N) {
        uint32_t a2 = aln[0];
#pragma unroll
        for (int q = 1; q < DBF_MAX_TERMS / 2; ++q)
          if (q == term / 2) a2 = aln[q];
        const uint16_t a_n = static_cast<uint16_t>(term & 1 ? a2 >> 16 : a2);
#pragma unroll
        for (int tok = 0; tok < TB; ++tok) {
          if constexpr (MODE == MODE_I8) {
            const int64_t tt = tok0 + tok;
            if (tt < p.T && p.s2_out) p.s2_out[(term * p.T + tt) * p.N + row] = acc[tok];
          }
          yacc[tok] += f16_bits_to_f32(a_n) * static_cast<float>(acc[tok]);
        }
      }
    }
    if (wv == 0 && row < p.N && p.y) {
#pragma unroll
      for (int tok = 0; tok < TB; ++tok) {
        const int64_t tt = tok0 + tok;
        if (tt < p.T) store_out(p.y, p.y_dtype, tt * p.ldy + row, yacc[tok], p.accumulate);
      }
    }
  }
  consumer_done(p.sync, ticket);
}

// ---- float consumers, wave by wave ----------------------------------------
// Wave wv of a stage-2 workgroup owns the K-blocks kb = wv, wv + NW, ... of
// B1 (ranks 32 KW kb ..).  Instead of the whole workgroup waiting for every
// producer, each wave waits only for the producers of its own ranks (their
// counter slots), then fetches its partials, builds its own tables and makes
// its lookups while other waves are still waiting.  Each wave accumulates
// only its own K-blocks, alpha of its row applied per term, and the waves
// are added in wave order at the end (reduce_waves), so the result does not
// depend on which wave finished first.
//
// Producer pid = ((tblk L + term) nrt2 + rt2) ks + split adds to counter
// slot pid % kSyncSlots; a wave waits until each slot of its producers
// holds that slot's full count (a superset of what it needs when several
// producers share a slot).  The reset rule of consumer_done needs every
// wait of the launch to be over before the last ticket: here the last wave
// of a workgroup to pass its final wait (counted in LDS) takes the
// workgroup's ticket.

// Wait until every producer of (tblk, term) whose rows fall in ranks
// [r0, r1) has published.  All lanes of the wave call it; bounded like
// wait_producers.
__device__ __forceinline__ void wait_ranks(const Sync& s, int tblk, int term, int L, int nrt2,
                                           int ks, int r0, int r1) {
  const int lane = threadIdx.x & 63;
  const int rt_lo = r0 / 64, rt_hi = min(nrt2, (r1 + 63) / 64);
  const int npid = (rt_hi - rt_lo) * ks;
  const unsigned ns = static_cast<unsigned>(kSyncSlots);
  const unsigned base = static_cast<unsigned>((tblk * L + term) * nrt2 + rt_lo) * ks;
  unsigned spins = 0;
  for (int j0 = 0; j0 < npid; j0 += 64) {
    const int j = j0 + lane;
    unsigned slot = 0, want = 0;
    if (j < npid) {
      // pids of consecutive (row tile, split) are consecutive
      slot = (base + static_cast<unsigned>(j)) % ns;
      want = s.n_prod / ns + (slot < s.n_prod % ns ? 1u : 0u);
    }
    unsigned have = 0;
    while (true) {
      if (have < want)
        have = __hip_atomic_load(s.slots + slot * kSyncStride, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_SYSTEM);
      if (__all(have >= want)) break;
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        if (lane == 0)
          __hip_atomic_fetch_or(s.ctr + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        break;
      }
    }
  }
}

// LDS operations of one wave are done in order; this keeps the compiler
// from moving them across the point and waits for this wave's own.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Splits of the first product the wave-by-wave consumers take (their
// partial loads are issued one item ahead, so they are held in registers).
constexpr int kWavesMaxKS = 2;

template <int TB, int KW, int NW>
__device__ __forceinline__ void stage2_role_waves(const Stage2& p, int64_t bid2, float* tbl,
                                                  float* red, unsigned* wg_ctr) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t tblk = bid2 / p.nrt;
  const int64_t rt = bid2 - tblk * p.nrt;
  const int64_t row = rt * 64 + lane;
  const int64_t nrt2 = layout_nrt(p.R);
  constexpr int G = 8 * KW;                       // groups of four ranks in a K-block
  constexpr int NE = (TB * G + 63) / 64;           // tables a lane builds
  float* wtbl = tbl + wv * (TB * G * 16);          // this wave's tables [TB][G][16]
  // this wave's items: (term, K-block wv + i NW) for every term, i < nmine
  const int nmine = wv < p.nkb ? static_cast<int>((p.nkb - 1 - wv) / NW) + 1 : 0;
  const int nitems = p.t.n * nmine;
  const int64_t tok0 = tblk * TB;
  // alpha of this lane's row for every term, two to a register (read before
  // the wait, by every lane with the row clamped)
  const int64_t arow = row < p.N ? row : p.N - 1;
  uint32_t aln[DBF_MAX_TERMS / 2];
#pragma unroll
  for (int q = 0; q < DBF_MAX_TERMS; q += 2) {
    const uint32_t lo = q < p.t.n ? p.t.alpha[q][arow] : 0x3C00u;
    const uint32_t hi = q + 1 < p.t.n ? p.t.alpha[q + 1][arow] : 0x3C00u;
    aln[q / 2] = lo | (hi << 16);
  }
  if (threadIdx.x == 0) wg_ctr[0] = 0u;
  // the sign words of this lane's row for item it
  auto words = [&](int it, uint32_t (&wd)[KW]) {
#pragma unroll
    for (int w = 0; w < KW; ++w) wd[w] = 0u;
    if (it < nitems) {
      const int term = it / nmine, i = it - term * nmine;
      load_row_words<KW>(p.t.b1[term] + ((rt * p.nkb + wv + static_cast<int64_t>(i) * NW) * 64 + lane) * KW, wd);
    }
  };
  uint32_t wd[KW];
  words(0, wd);
  __syncthreads();  // wg_ctr cleared
  // wait for every producer of this wave's ranks, all terms
  if (nmine > 0) {
    const int r0 = wv * 32 * KW;
    const int r1 = static_cast<int>(min(p.R, static_cast<int64_t>(wv + (nmine - 1) * NW + 1) * 32 * KW));
    for (int term = 0; term < p.t.n; ++term)
      wait_ranks(p.sync, static_cast<int>(tblk), term, p.t.n, static_cast<int>(nrt2), p.ks, r0, r1);
  }
  // the partials of item it, as raw system-scope loads (at most kWavesMaxKS
  // splits), addresses clamped past R and T
  struct Raw {
    float4 q[NE][kWavesMaxKS];
  };
  auto issue = [&](int it, Raw& r) {
    const int term = it < nitems ? it / nmine : 0, i = it < nitems ? it - term * nmine : 0;
    const int64_t kbase = (wv + static_cast<int64_t>(i) * NW) * 32 * KW;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int ent = lane + 64 * e;
      const int tok = ent / G, g = ent - tok * G;
      const int64_t tt = tok0 + tok, k = kbase + 4 * g;
      const bool in = it < nitems && ent < TB * G && tt < p.T && k < p.R;
      const int64_t base = (static_cast<int64_t>(term) * p.ks * p.T + (in ? tt : 0)) * p.rs + (in ? k : 0);
#pragma unroll
      for (int sp = 0; sp < kWavesMaxKS; ++sp)
        r.q[e][sp] = sp < p.ks ? load_shared4<float4>(static_cast<const float*>(p.ws) + base + sp * p.T * p.rs)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  Raw raw;
  issue(0, raw);
  if (lane == 0) {
    // this wave's waits are over; the workgroup's last such wave takes the
    // ticket, after its first partials' loads (a wave's loads return in
    // order, so those need not wait for the ticket's round trip)
    const unsigned done = __hip_atomic_fetch_add(wg_ctr, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP);
    if (done == NW - 1) wg_ctr[1] = take_ticket_any(p.sync);
  }
  float yacc[TB], acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) yacc[t] = acc[t] = 0.f;
  for (int it = 0; it < nitems; ++it) {
    const int term = it / nmine, i = it - term * nmine;
    const int64_t kbase = (wv + static_cast<int64_t>(i) * NW) * 32 * KW;
    // this item's w (splits summed in order; zeros past R or T)
    float v[NE][4];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      float4 sm = raw.q[e][0];
#pragma unroll
      for (int sp = 1; sp < kWavesMaxKS; ++sp)
        if (sp < p.ks) {
          sm.x += raw.q[e][sp].x; sm.y += raw.q[e][sp].y; sm.z += raw.q[e][sp].z; sm.w += raw.q[e][sp].w;
        }
      const int ent = lane + 64 * e;
      const int tok = ent / G, g = ent - tok * G;
      const int64_t k = kbase + 4 * g;
      const bool in = tok0 + tok < p.T;
      v[e][0] = in && k < p.R ? sm.x : 0.f;
      v[e][1] = in && k + 1 < p.R ? sm.y : 0.f;
      v[e][2] = in && k + 2 < p.R ? sm.z : 0.f;
      v[e][3] = in && k + 3 < p.R ? sm.w : 0.f;
    }
    // the next item's partials and sign words, before this item's lookups
    // (none past the last item: loads still in flight would hold the wave)
    uint32_t wdn[KW];
#pragma unroll
    for (int w = 0; w < KW; ++w) wdn[w] = 0u;
    if (it + 1 < nitems) {
      issue(it + 1, raw);
      words(it + 1, wdn);
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int ent = lane + 64 * e;
      if (ent < TB * G) {
        const int tok = ent / G, g = ent - tok * G;
        build_signed16<float>(v[e][0], v[e][1], v[e][2], v[e][3], wtbl + (tok * G + g) * 16,
                              tok * G + g);
      }
    }
    wave_lds_sync();
    float acc2[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) acc2[t] = 0.f;
#pragma unroll
    for (int w = 0; w < KW; ++w) {
#pragma unroll
      for (int c = 0; c < 8; c += 2) {
        const int n0 = (wd[w] >> (4 * c)) & 15, n1 = (wd[w] >> (4 * c + 4)) & 15;
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          acc[t] += wtbl[(t * G + w * 8 + c) * 16 + n0];
          acc2[t] += wtbl[(t * G + w * 8 + c + 1) * 16 + n1];
        }
      }
    }
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] += acc2[t];
    wave_lds_sync();  // lookups done before the tables are rebuilt
#pragma unroll
    for (int w = 0; w < KW; ++w) wd[w] = wdn[w];
    if (i == nmine - 1) {
      // the term's last K-block of this wave: alpha of the row, then on
      uint32_t a2 = aln[0];
#pragma unroll
      for (int q = 1; q < DBF_MAX_TERMS / 2; ++q)
        if (q == term / 2) a2 = aln[q];
      const float al = f16_bits_to_f32(static_cast<uint16_t>(term & 1 ? a2 >> 16 : a2));
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        yacc[t] += al * acc[t];
        acc[t] = 0.f;
      }
    }
  }
  reduce_waves<float, TB, NW>(red, yacc);
  if (wv == 0 && row < p.N && p.y) {
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const int64_t tt = tok0 + t;
      if (tt < p.T) store_out(p.y, p.y_dtype, tt * p.ldy + row, yacc[t], p.accumulate);
    }
  }
  consumer_done(p.sync, wg_ctr[1]);
}

// NW waves per workgroup (16 or 8; the launcher picks, see pick_waves).
// CW: float consumers wave by wave (stage2_role_waves).
template <typename A, int TB, int KW1, int KW2, int MODE, int NW, bool CW = false>
__global__ void __launch_bounds__(64 * NW) decode_kernel(Stage1 s1, Stage2 s2, int n1,
                                                         int run_stage2) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int KWM = KW1 > KW2 ? KW1 : KW2;
  A* tbl = reinterpret_cast<A*>(smem);
  A* red = tbl + tbl_elems<TB, KWM, NW>();
  const int bid = blockIdx.x;
  if (bid < n1) {
    stage1_role<A, TB, KW1, MODE, NW>(s1, bid, tbl, red);
    if (run_stage2) publish(s2.sync, static_cast<unsigned>(bid));
    return;
  }
  if constexpr (CW) {
    static_assert(MODE == MODE_F && TB <= 2, "wave-by-wave consumers: float, up to two tokens");
    // two words after the tables and wave partials: the workgroup's count of
    // waves past their last wait, and its ticket
    unsigned* wg_ctr = reinterpret_cast<unsigned*>(red + red_elems<TB, NW>());
    stage2_role_waves<TB, KW2, NW>(s2, bid - n1, tbl, red, wg_ctr);
  } else {
    stage2_role<A, TB, KW2, MODE, NW>(s2, bid - n1, tbl, red);
  }
}

// Stage 1 aims at about this many waves (512 workgroups of 8, 256 of 16).
constexpr int64_t kStage1Waves = 4096;

// Waves per decode workgroup for a launch whose 16-wave stage 1 is `a16`
// with n1_16 workgroups.  Sixteen halve each lane's lookups per 64-row tile
// and the partials, but a CU then holds one workgroup instead of three, so
// they pay only while stage 1 still splits K and fits the 256 CUs at once,
// or when R is large enough that stage 2 dominates (two_stage).  Measured,
// 16 vs 8 waves (us): 4096^2 R 2048 at 4 / 16 tokens 11.6 / 18.7 vs 12.7 /
// 21.0, at 32 tokens 31.4 vs 29.2; three terms of 11008 x 4096 at 1 / 4
// tokens 14.5 / 31.1 vs 16.2 / 30.3; 8192^2 R 6144 at 4 / 8 tokens 27.0 /
// 44.8 vs 29.6 / 52.7; boolean kernels 2 x 4096^2 at 1 / 8 tokens 8.7 / 18.1
// vs 9.3 / 16.9, 3 x 11008 x 4096 at 1 token 16.4 vs 15.6.
int pick_waves(const lut::Stage1& a16, int64_t n1_16, int64_t R, bool two_stage) {
  // a launch with no stage 2 gains only the halved partials, and fewer than
  // 128 workgroups would leave half the CUs idle (the backward's one-token
  // products on 2048-row matrices: 39.1 vs 37.4 us per backward)
  if (!two_stage && n1_16 < 128) return 8;
  if (a16.ks >= 2 && n1_16 <= 256) return 16;
  if (two_stage && R >= 4096) return 16;
  return 8;
}

// ---- boolean kernels (Multi-Boolean form) -------------------------------
// The stage-1 role alone computes s_out . (Wb (s_in . x)) for each kernel
// (Wb in the place of B2, s_in of gamma, s_out of beta, N rows), as K-split
// partials; consumer workgroups then sum the partials of every kernel and
// split into y.
struct SumArgs {
  int L, ks;
  int64_t T, N, rs;
  const float* ws;  // partials [L][ks][T][rs]
  void* y;
  int y_dtype;
  int64_t ldy;
  int accumulate;
  Sync sync;
  int64_t nrt;  // row tiles of N; consumer = (token block, row tile)
};

// Consumer `bid2`: 64 rows (lane) x TB tokens (wave).  Every partial of a
// (row, token) is loaded before the sum, which runs in (kernel, split) order.
template <int TB>
__device__ __forceinline__ void sum_role(const SumArgs& p, int64_t bid2) {
  const int64_t tblk = bid2 / p.nrt;
  const int64_t rt = bid2 - tblk * p.nrt;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  wait_producers(p.sync, false);  // partials via system-scope loads
  unsigned ticket = 0;
  bool took = false;
  const int64_t row = rt * 64 + lane, tt = tblk * TB + wv;
  if (wv < TB && row < p.N && tt < p.T) {
    const int np = p.L * p.ks;
    const uint32_t* base = reinterpret_cast<const uint32_t*>(p.ws) + tt * p.rs + row;
    float s = 0.f;
    for (int j0 = 0; j0 < np; j0 += 16) {
      uint32_t q[16];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        q[j] = j0 + j < np ? __hip_atomic_load(base + (j0 + j) * p.T * p.rs, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_SYSTEM)
                           : 0u;
      // after the first partials' loads, so its round trip overlaps them
      if (!took) {
        ticket = take_ticket(p.sync);
        took = true;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j0 + j < np) s += __uint_as_float(q[j]);
    }
    store_out(p.y, p.y_dtype, tt * p.ldy + row, s, p.accumulate);
  }
  if (!took) ticket = take_ticket(p.sync);
  consumer_done(p.sync, ticket);
}

template <int TB, int KW, int NW>
__global__ void __launch_bounds__(64 * NW) bool_decode_kernel(Stage1 s1, SumArgs s2, int n1) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* tbl = reinterpret_cast<float*>(smem);
  float* red = tbl + tbl_elems<TB, KW, NW>();
  const int bid = blockIdx.x;
  if (bid < n1) {
    stage1_role<float, TB, KW, MODE_F, NW>(s1, bid, tbl, red);
    publish(s2.sync, static_cast<unsigned>(bid));
    return;
  }
  sum_role<TB>(s2, bid - n1);
}

template <typename A, int MODE, int NW>
hipError_t run(const Stage1& s1, const Stage2& s2, int n1, int n2, int run_stage2,
               int tb, int kw1, int kw2, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(n1 + (run_stage2 ? n2 : 0));
  // Float consumers wave by wave for one or two tokens of layers with whole
  // 128-feature K-blocks (stage2_role_waves).
  if constexpr (MODE == MODE_F) {
    if (run_stage2 && tb <= 2 && kw1 == 4 && kw2 == 4 && s2.ks <= kWavesMaxKS &&
        s2.t.n == 1 && s2.nkb <= NW) {
      const size_t lds = (tb == 1 ? lds_bytes<A, 1, 4, NW>() : lds_bytes<A, 2, 4, NW>()) + 16;
      if (tb == 1)
        decode_kernel<A, 1, 4, 4, MODE, NW, true><<<dim3(grid), 64 * NW, lds, s>>>(s1, s2, n1, run_stage2);
      else
        decode_kernel<A, 2, 4, 4, MODE, NW, true><<<dim3(grid), 64 * NW, lds, s>>>(s1, s2, n1, run_stage2);
      return hipGetLastError();
    }
  }
#define DBF_LAUNCH(TB_, K1_, K2_)                                                        \
  decode_kernel<A, TB_, K1_, K2_, MODE, NW>                                              \
      <<<dim3(grid), 64 * NW, lds_bytes<A, TB_, (K1_ > K2_ ? K1_ : K2_), NW>(), s>>>(     \
          s1, s2, n1, run_stage2)
#define DBF_K2(TB_, K1_)                     \
  switch (kw2) {                             \
    case 1: DBF_LAUNCH(TB_, K1_, 1); break;  \
    case 2: DBF_LAUNCH(TB_, K1_, 2); break;  \
    case 3: DBF_LAUNCH(TB_, K1_, 3); break;  \
    default: DBF_LAUNCH(TB_, K1_, 4); break; \
  }
#define DBF_K1(TB_)                \
  switch (kw1) {                   \
    case 1: DBF_K2(TB_, 1); break; \
    case 2: DBF_K2(TB_, 2); break; \
    case 3: DBF_K2(TB_, 3); break; \
    default: DBF_K2(TB_, 4); break; \
  }
  switch (tb) {
    case 1: DBF_K1(1); break;
    case 2: DBF_K1(2); break;
    default: DBF_K1(4); break;
  }
#undef DBF_K1
#undef DBF_K2
#undef DBF_LAUNCH
  return hipGetLastError();
}

Stage2 make_stage2(const TermPtrs& t, const Stage1& s1, int64_t N, int64_t R, int64_t T,
                   void* ws, int n1) {
  Stage2 b{};
  b.t = t; b.T = T; b.N = N; b.R = R; b.nkb = layout_nkb(R); b.ks = s1.ks;
  b.ws = s1.ws; b.rs = s1.rs;
  b.nrt = layout_nrt(N);
  b.n2 = static_cast<unsigned>(b.nrt * s1.ntb);
  b.sync = make_sync(ws, n1, b.n2);
  return b;
}

}  // namespace

lut::Stage1 make_stage1(const TermPtrs& t, int64_t M, int64_t R, const void* x, int x_dtype,
                        int64_t T, int64_t ldx, void* ws, bool split, int* n1, int nw) {
  lut::Stage1 a{};
  a.t = t; a.x = x; a.x_dtype = x_dtype; a.ldx = ldx; a.T = T; a.M = M; a.R = R;
  a.nkb = layout_nkb(M);
  a.nrt = layout_nrt(R);
  int64_t per = 0;
  a.ntb = static_cast<int>((T + lut::pick_tb(T) - 1) / lut::pick_tb(T));
  a.ks = lut::pick_ks(a.nrt * a.ntb, t.n, a.nkb, split ? kStage1Waves / nw : 1, &per, nw);
  a.kb_per_split = per;
  a.rs = ws_rstride(R);
  // four 16-bit activations per 8-byte load (fp32 input takes the bounded path)
  a.vec4 = (x_dtype != DBF_F32) && (ldx % 4 == 0) && (reinterpret_cast<uintptr_t>(x) % 8 == 0) &&
           (M % 4 == 0);
  for (int i = 0; i < t.n; ++i)
    if (t.gamma[i] && reinterpret_cast<uintptr_t>(t.gamma[i]) % 8 != 0) a.vec4 = 0;
  *n1 = static_cast<int>(a.nrt * a.ks * t.n * a.ntb);
  a.ws = static_cast<unsigned char*>(ws) + kWsHeadBytes;
  return a;
}

size_t decode_ws_bytes(int64_t /*N*/, int64_t M, int64_t R, int n_terms, int64_t T) {
  int64_t per = 0;
  const int64_t ntb = (T + lut::pick_tb(T) - 1) / lut::pick_tb(T);
  // the most splits any call of these sizes picks: split or not, with the
  // decode kernels' workgroups or the adapter kernels' 8-wave ones
  int ks = 1;
  for (const int nw : {lut::kWaves, 8})
    ks = std::max({ks,
                   lut::pick_ks(layout_nrt(R) * ntb, n_terms, layout_nkb(M), kStage1Waves / nw, &per, nw),
                   lut::pick_ks(layout_nrt(R) * ntb, n_terms, layout_nkb(M), 1, &per, nw)});
  return kWsHeadBytes + static_cast<size_t>(n_terms) * ks * static_cast<size_t>(T) *
                                   static_cast<size_t>(ws_rstride(R)) * 4u;
}

hipError_t launch_decode(const TermPtrs& t, int64_t N, int64_t M, int64_t R,
                         const void* x, int x_dtype, int64_t T, int64_t ldx,
                         void* y, int y_dtype, int64_t ldy, int accumulate,
                         void* ws, hipStream_t s) {
  int n1 = 0;
  Stage1 a = make_stage1(t, M, R, x, x_dtype, T, ldx, ws, true, &n1, 16);
  const int nw = pick_waves(a, n1, R, true);
  if (nw != 16) a = make_stage1(t, M, R, x, x_dtype, T, ldx, ws, true, &n1, nw);
  Stage2 b = make_stage2(t, a, N, R, T, ws, n1);
  b.y = y; b.y_dtype = y_dtype; b.ldy = ldy; b.accumulate = accumulate;
  const int kw1 = static_cast<int>(layout_kw(M)), kw2 = static_cast<int>(layout_kw(R));
  if (nw == 16)
    return run<float, MODE_F, 16>(a, b, n1, static_cast<int>(b.n2), 1, pick_tb(T), kw1, kw2, s);
  return run<float, MODE_F, 8>(a, b, n1, static_cast<int>(b.n2), 1, pick_tb(T), kw1, kw2, s);
}

hipError_t launch_bool_decode(const TermPtrs& t, int64_t N, int64_t M, const void* x,
                              int x_dtype, int64_t T, int64_t ldx, void* y, int y_dtype,
                              int64_t ldy, int accumulate, void* ws, hipStream_t s) {
  int n1 = 0;
  Stage1 a = make_stage1(t, M, N, x, x_dtype, T, ldx, ws, true, &n1, 16);
  const int nw = pick_waves(a, n1, 0, false);
  if (nw != 16) a = make_stage1(t, M, N, x, x_dtype, T, ldx, ws, true, &n1, nw);
  SumArgs b{};
  b.L = t.n; b.ks = a.ks; b.T = T; b.N = N; b.rs = a.rs;
  b.ws = static_cast<const float*>(a.ws);
  b.y = y; b.y_dtype = y_dtype; b.ldy = ldy; b.accumulate = accumulate;
  b.nrt = layout_nrt(N);
  const int n2 = static_cast<int>(b.nrt * a.ntb);
  b.sync = make_sync(ws, n1, n2);
  const unsigned grid = static_cast<unsigned>(n1 + n2);
  const int tb = pick_tb(T), kw = static_cast<int>(layout_kw(M));
#define DBF_BOOL(TB_, KW_, NW_)                                                         \
  bool_decode_kernel<TB_, KW_, NW_>                                                     \
      <<<dim3(grid), 64 * NW_, lds_bytes<float, TB_, KW_, NW_>(), s>>>(a, b, n1)
#define DBF_BOOL_KW(TB_, NW_)              \
  switch (kw) {                            \
    case 1: DBF_BOOL(TB_, 1, NW_); break;  \
    case 2: DBF_BOOL(TB_, 2, NW_); break;  \
    case 3: DBF_BOOL(TB_, 3, NW_); break;  \
    default: DBF_BOOL(TB_, 4, NW_); break; \
  }
#define DBF_BOOL_TB(NW_)                \
  switch (tb) {                         \
    case 1: DBF_BOOL_KW(1, NW_); break; \
    case 2: DBF_BOOL_KW(2, NW_); break; \
    default: DBF_BOOL_KW(4, NW_); break; \
  }
  if (nw == 16) {
    DBF_BOOL_TB(16)
  } else {
    DBF_BOOL_TB(8)
  }
#undef DBF_BOOL_TB
#undef DBF_BOOL_KW
#undef DBF_BOOL
  return hipGetLastError();
}

hipError_t launch_decode_i8(const TermPtrs& t, int64_t N, int64_t M, int64_t R,
                            const int8_t* x, int64_t T, int64_t ldx,
                            int32_t* s1, int32_t* s2, void* y, int y_dtype,
                            int64_t ldy, void* ws, hipStream_t s) {
  int n1 = 0;
  // eight waves: the int8 variant is not timed against the float path
  const Stage1 a = make_stage1(t, M, R, x, DBF_I8, T, ldx, ws, false, &n1, 8);
  Stage2 b = make_stage2(t, a, N, R, T, ws, n1);
  b.y = y; b.y_dtype = y_dtype; b.ldy = ldy; b.accumulate = 0; b.s2_out = s2;
  b.s1_out = s1;
  const int run2 = 1;  // stage 2 also sums the K-split partials into s1
  const int tb = pick_tb(T), kw1 = static_cast<int>(layout_kw(M)),
            kw2 = static_cast<int>(layout_kw(R));
  if (t.beta[0] == nullptr)
    return run<int32_t, MODE_I8, 8>(a, b, n1, static_cast<int>(b.n2), run2, tb, kw1, kw2, s);
  return run<float, MODE_I8_BETA, 8>(a, b, n1, static_cast<int>(b.n2), run2, tb, kw1, kw2, s);
}

}  // namespace dbf
