// Device building blocks of the sign-accumulate over packed bits with
// 16-entry signed subset-sum tables, shared by the decode kernel and the
// fused adapter kernel.
//
// For each group of four consecutive activations a0..a3 and each 4-bit
// pattern n the table holds
//     E[n] = sum_j (bit j of n ? +a_j : -a_j) = 2 * sum_{bit j set} a_j - sum_j a_j,
// the identity  sum_k s_k a_k = 2 sum_{s_k=+1} a_k - sum_k a_k  applied per
// group with the -sum folded into every entry, so a row's product with the
// activations is one LDS lookup and one add per nibble of its packed bits
// (LoRDBA section 2, "Kernel de Inferencia": additions and subtractions in
// place of multiplications in the inner products).
//
// A workgroup is NW wavefronts over one 64-row tile (16 in the decode
// kernels, 8 in the adapter kernels); lane = row.  A pass covers NW * PW
// K-blocks; wave wv takes blocks kp + j * NW + wv (j < PW), so every wave
// reads whole contiguous tiles and all 64 lanes of a wave look up the same
// group's 16 entries together (16 LDS banks, no conflicts).
#pragma once

#include "dbf_internal.h"

namespace dbf {
namespace lut {

// Waves per workgroup: the templates' default, 16.  The decode launchers
// pick 16 or 8 per launch (pick_waves in dbf_decode.hip); the adapter
// kernels use 8 (their row roles need more than the 128 registers a
// 1024-thread workgroup leaves a wave).
constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxKS = 8;
constexpr unsigned kSpinLimit = 1u << 26;

enum { MODE_F = 0, MODE_I8_BETA = 1, MODE_I8 = 2 };

// Token-block size and K-blocks per wave per pass for T tokens.
__host__ __device__ constexpr int pw_of(int tb) { return tb == 1 ? 2 : 1; }
inline int pick_tb(int64_t T) { return T <= 1 ? 1 : (T <= 4 ? 2 : 4); }

// LDS (elements of type A): tables [TB][groups][16], wave partials
// [4][TB][64].
template <int TB, int KW, int NW = kWaves>
__host__ __device__ constexpr int tbl_elems() { return TB * NW * pw_of(TB) * 8 * KW * 16; }
template <int TB, int NW = kWaves>
__host__ __device__ constexpr int red_elems() { return NW * TB * 64; }
template <typename A, int TB, int KW, int NW = kWaves>
__host__ __device__ constexpr size_t lds_bytes() {
  return sizeof(A) * (tbl_elems<TB, KW, NW>() + red_elems<TB, NW>());
}

// A result another workgroup of the launch will read: written through to
// memory (system-scope store), so the producer needs no L2 writeback.
template <typename V>
__device__ __forceinline__ void store_shared(V* p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Four results of other workgroups of the launch (16-byte aligned), read at
// system scope: the loads bypass the caches, so they see what store_shared
// wrote through once the producer's counter was seen, without an
// invalidation of the whole L2.
template <typename V4, typename E>
__device__ __forceinline__ V4 load_shared4(const E* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  V4 v;
  v.x = __builtin_bit_cast(E, static_cast<uint32_t>(lo));
  v.y = __builtin_bit_cast(E, static_cast<uint32_t>(lo >> 32));
  v.z = __builtin_bit_cast(E, static_cast<uint32_t>(hi));
  v.w = __builtin_bit_cast(E, static_cast<uint32_t>(hi >> 32));
  return v;
}

// The 16 entries of group gi of a table, E[n] = P[n % 4] + Q[n / 4], written
// at e = tbl + 16 gi as four 16-byte chunks (entries 4 j .. 4 j + 3 = chunk j).
// Consecutive lanes build consecutive groups, 64 bytes apart, so chunk j of
// every lane would fall on the same few banks: each lane writes its chunks in
// the order j = (c + rot(gi)) % 4, c = 0..3, with rot(gi) = (gi / 2 + gi / 8)
// % 4.  Any 8 (16) consecutive groups then cover 8 (16) distinct 16-byte bank
// slots of 32 (64) banks per write, and the layout the lookups read is the
// plain one.
template <typename A>
__device__ __forceinline__ void build_signed16(A a0, A a1, A a2, A a3, A* e, int gi) {
  typedef A A4 __attribute__((ext_vector_type(4)));
  const A p0 = -a0 - a1, p1 = a0 - a1, p2 = a1 - a0, p3 = a0 + a1;
  const A q0 = -a2 - a3, q1 = a2 - a3, q2 = a3 - a2, q3 = a2 + a3;
  const int rot = ((gi >> 1) + (gi >> 3)) & 3;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int j = (c + rot) & 3;
    const A q = (j & 2) ? ((j & 1) ? q3 : q2) : ((j & 1) ? q1 : q0);
    A4 v;
    v.x = p0 + q; v.y = p1 + q; v.z = p2 + q; v.w = p3 + q;
    *reinterpret_cast<A4*>(e + 4 * j) = v;
  }
}

template <int KW>
__device__ __forceinline__ void load_row_words(const uint32_t* p, uint32_t* wd) {
  if constexpr (KW == 4) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    wd[0] = v[0]; wd[1] = v[1]; wd[2] = v[2]; wd[3] = v[3];
  } else if constexpr (KW == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    wd[0] = v.x; wd[1] = v.y;
  } else {
#pragma unroll
    for (int w = 0; w < KW; ++w) wd[w] = p[w];
  }
}

// This lane's words of the pass starting at K-block kp (zeros past kb_end).
template <int TB, int KW, int NW = kWaves>
__device__ __forceinline__ void load_pass_bits(const uint32_t* __restrict__ bits,
                                               int64_t rt, int64_t nkb, int64_t kp,
                                               int64_t kb_end,
                                               uint32_t (&wd)[pw_of(TB)][KW]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < pw_of(TB); ++j) {
    const int64_t kb = kp + j * NW + wv;
#pragma unroll
    for (int w = 0; w < KW; ++w) wd[j][w] = 0;
    if (kb < kb_end) load_row_words<KW>(bits + ((rt * nkb + kb) * 64 + lane) * KW, wd[j]);
  }
}

// Table entries of a pass, [TB][ng] (ng groups of four activations per
// token), and how many of them one thread builds.
template <int TB, int KW, int NW = kWaves>
__host__ __device__ constexpr int ents_per_thread() {
  return (TB * NW * pw_of(TB) * 8 * KW + 64 * NW - 1) / (64 * NW);
}

// The four activations of each table entry this thread builds (entry
// threadIdx.x + i * kThreads; act4(tok, g, a) writes group g's four values).
// Vector loads return in order within a wave, so a caller issues these loads
// before loads whose data it needs later (the pass's sign words), and the
// table build need not wait for those.
template <typename A, int TB, int KW, int NW = kWaves, typename Act4>
__device__ __forceinline__ void load_acts(Act4 act4, int ng,
                                          A (&v)[ents_per_thread<TB, KW, NW>()][4]) {
#pragma unroll
  for (int i = 0; i < ents_per_thread<TB, KW, NW>(); ++i) {
    const int e = threadIdx.x + i * 64 * NW;
    if (e < TB * ng) {
      const int tok = e / ng, g = e - tok * ng;
      act4(tok, g, v[i]);
    }
  }
}

// Tables for the groups of the pass built from the loaded activations
// straight into LDS, then this lane's lookups of the pass: acc[tok] += sum
// over the pass of S[row, k] * act[tok][k].  Two accumulators per token keep
// the adds of consecutive nibbles independent, so many LDS reads are in
// flight.  Ends with a barrier, so the tables may be overwritten afterwards.
template <typename A, int TB, int KW, int NW = kWaves>
__device__ __forceinline__ void tables_and_lookups_v(
    const A (&v)[ents_per_thread<TB, KW, NW>()][4], A* tbl, int ng, int64_t kp, int64_t kb_end,
    const uint32_t (&wd)[pw_of(TB)][KW], A* acc) {
  constexpr int PW = pw_of(TB);
  constexpr int gpp = NW * PW * 8 * KW;
  const int wv = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < ents_per_thread<TB, KW, NW>(); ++i) {
    const int e = threadIdx.x + i * 64 * NW;
    if (e < TB * ng) {
      const int tok = e / ng, g = e - tok * ng;
      build_signed16<A>(v[i][0], v[i][1], v[i][2], v[i][3], tbl + (tok * gpp + g) * 16, tok * gpp + g);
    }
  }
  __syncthreads();
  A acc2[TB];
#pragma unroll
  for (int tok = 0; tok < TB; ++tok) acc2[tok] = A(0);
#pragma unroll
  for (int j = 0; j < PW; ++j) {
    if (kp + j * NW + wv >= kb_end) continue;  // wave-uniform
    const A* tb = tbl + ((j * NW + wv) * 8 * KW) * 16;
#pragma unroll
    for (int w = 0; w < KW; ++w) {
#pragma unroll
      for (int c = 0; c < 8; c += 2) {
        const int n0 = (wd[j][w] >> (4 * c)) & 15;
        const int n1 = (wd[j][w] >> (4 * c + 4)) & 15;
#pragma unroll
        for (int tok = 0; tok < TB; ++tok) {
          acc[tok] += tb[(tok * gpp + w * 8 + c) * 16 + n0];
          acc2[tok] += tb[(tok * gpp + w * 8 + c + 1) * 16 + n1];
        }
      }
    }
  }
#pragma unroll
  for (int tok = 0; tok < TB; ++tok) acc[tok] += acc2[tok];
  __syncthreads();
}

template <typename A, int TB, int KW, int NW = kWaves, typename Act4>
__device__ __forceinline__ void tables_and_lookups(Act4 act4, A* tbl, int ng, int64_t kp,
                                                   int64_t kb_end,
                                                   const uint32_t (&wd)[pw_of(TB)][KW],
                                                   A* acc) {
  A v[ents_per_thread<TB, KW, NW>()][4];
  load_acts<A, TB, KW, NW>(act4, ng, v);
  tables_and_lookups_v<A, TB, KW, NW>(v, tbl, ng, kp, kb_end, wd, acc);
}

// Sum of the NW wave partials of each lane's row, in wave order; the result
// is valid in wave 0.
template <typename A, int TB, int NW = kWaves>
__device__ __forceinline__ void reduce_waves(A* red, A* acc) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int tok = 0; tok < TB; ++tok) red[(wv * TB + tok) * 64 + lane] = acc[tok];
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int tok = 0; tok < TB; ++tok) {
      A s = red[tok * 64 + lane];
#pragma unroll
      for (int v = 1; v < NW; ++v) s += red[(v * TB + tok) * 64 + lane];
      acc[tok] = s;
    }
  }
  __syncthreads();
}

// ---- stage 1: w = beta . (B2 (gamma . x)) over one row tile and K split ----
struct Stage1 {
  TermPtrs t;
  const void* x;
  int x_dtype;
  int64_t ldx, T, M, R;
  int64_t nkb, kb_per_split, nrt;
  int ks;
  int ntb;        // token blocks (of TB tokens), one per workgroup
  void* ws;       // partials [L][ks][T][rs]
  int64_t rs;
  int vec4;       // x rows allow 8-byte loads of four activations
};

// Where stage 1 takes a term's B2, gamma and beta from: the term table of
// the launch, or (OneTerm) a single term's pointers, e.g. the adapter of a
// workgroup's token.
struct TermSrc {
  const TermPtrs& t;
  __device__ const uint32_t* b2(int i) const { return t.b2[i]; }
  __device__ const uint16_t* gamma(int i) const { return t.gamma[i]; }
  __device__ const uint16_t* beta(int i) const { return t.beta[i]; }
  __device__ int n() const { return t.n; }
};
struct OneTerm {
  const uint32_t* b2_;
  const uint16_t* gamma_;
  const uint16_t* beta_;
  __device__ const uint32_t* b2(int) const { return b2_; }
  __device__ const uint16_t* gamma(int) const { return gamma_; }
  __device__ const uint16_t* beta(int) const { return beta_; }
  __device__ int n() const { return 1; }
};

// Stage-1 workgroup `bid` in [0, ntb * L * nrt * ks): its token block, term,
// row tile of B2 and K-blocks [kb0, kb1) of its split (one or more passes).
template <typename A, int TB, int KW, int MODE, int NW = kWaves, class Src = TermSrc>
__device__ __forceinline__ void stage1_role_src(const Stage1& p, const Src& src, int bid, A* tbl,
                                                A* red) {
  constexpr int PW = pw_of(TB);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int per_term = static_cast<int>(p.nrt) * p.ks;
  const int per_tb = src.n() * per_term;
  const int tblk = bid / per_tb;
  bid -= tblk * per_tb;
  const int term = bid / per_term;
  const int rem = bid - term * per_term;
  const int64_t rt = rem / p.ks;
  const int split = rem - static_cast<int>(rt) * p.ks;
  const int64_t kb0 = static_cast<int64_t>(split) * p.kb_per_split;
  const int64_t kb1 = min(p.nkb, kb0 + p.kb_per_split);
  const uint32_t* bits = src.b2(term);
  const uint16_t* gam = src.gamma(term);
  const int64_t row = rt * 64 + lane;
  const int64_t tok0 = static_cast<int64_t>(tblk) * TB;

  // beta of the rows this workgroup stores, read first: an input, and a
  // wave's loads return in order.  Every lane loads (row clamped), so no
  // branch holds the load, and the value is converted only where it is used.
  uint16_t bet = 0;
  if constexpr (MODE == MODE_F) bet = src.beta(term)[row < p.R ? row : p.R - 1];
  uint32_t wd[PW][KW];
  A acc[TB];
#pragma unroll
  for (int i = 0; i < TB; ++i) acc[i] = A(0);
  for (int64_t kp = kb0; kp < kb1; kp += NW * PW) {
    const int64_t kb_end = min(kb1, kp + NW * PW);
    const int64_t k0 = kp * 32 * KW;
    const int ng = static_cast<int>((kb_end - kp) * 8 * KW);
    auto act4 = [&](int tok, int g, A* a) {
      const int64_t tt = tok0 + tok, k = k0 + 4 * g;
      if constexpr (MODE == MODE_F) {
        if (p.vec4) {
          // M % 4 == 0: a group is wholly in or out.  Both loads are issued
          // by every lane (indices clamped), out-of-range groups give zeros.
          const bool in = tt < p.T && k < p.M;
          const int64_t tc = in ? tt : 0, kc = in ? k : 0;
          const uint2 xv = *reinterpret_cast<const uint2*>(
              static_cast<const uint16_t*>(p.x) + tc * p.ldx + kc);
          const uint2 gv = *reinterpret_cast<const uint2*>(gam + kc);
          const uint16_t xs[4] = {uint16_t(xv.x), uint16_t(xv.x >> 16), uint16_t(xv.y),
                                  uint16_t(xv.y >> 16)};
          const uint16_t gs[4] = {uint16_t(gv.x), uint16_t(gv.x >> 16), uint16_t(gv.y),
                                  uint16_t(gv.y >> 16)};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float xf = p.x_dtype == DBF_BF16 ? bf16_bits_to_f32(xs[j]) : f16_bits_to_f32(xs[j]);
            a[j] = in ? f16_bits_to_f32(gs[j]) * xf : 0.f;
          }
          return;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        A v = A(0);
        if (tt < p.T && k + j < p.M) {
          if constexpr (MODE == MODE_F)
            v = f16_bits_to_f32(gam[k + j]) * load_act(p.x, p.x_dtype, tt * p.ldx + k + j);
          else
            v = static_cast<const int8_t*>(p.x)[tt * p.ldx + k + j];
        }
        a[j] = v;
      }
    };
    // the pass's sign words, then its activations, all in flight together
    // (the activations are converted as they arrive, so loads issued after
    // them would wait for them)
    load_pass_bits<TB, KW, NW>(bits, rt, p.nkb, kp, kb1, wd);
    A v[ents_per_thread<TB, KW, NW>()][4];
    load_acts<A, TB, KW, NW>(act4, ng, v);
    tables_and_lookups_v<A, TB, KW, NW>(v, tbl, ng, kp, kb_end, wd, acc);
  }
  reduce_waves<A, TB, NW>(red, acc);
  if (wv == 0 && row < p.R) {
#pragma unroll
    for (int tok = 0; tok < TB; ++tok) {
      const int64_t tt = tok0 + tok;
      if (tt < p.T) {
        const int64_t o = ((static_cast<int64_t>(term) * p.ks + split) * p.T + tt) * p.rs + row;
        if constexpr (MODE == MODE_F)
          store_shared(static_cast<float*>(p.ws) + o, f16_bits_to_f32(bet) * acc[tok]);
        else
          store_shared(static_cast<int32_t*>(p.ws) + o, static_cast<int32_t>(acc[tok]));
      }
    }
  }
}

template <typename A, int TB, int KW, int MODE, int NW = kWaves>
__device__ __forceinline__ void stage1_role(const Stage1& p, int bid, A* tbl, A* red) {
  stage1_role_src<A, TB, KW, MODE, NW>(p, TermSrc{p.t}, bid, tbl, red);
}

// ---- handoff between the two roles of a launch ---------------------------
// Producer p adds one to counter p % kSyncSlots in the workspace head, each
// counter in its own 256-byte slot.  Its results are written through to
// memory first (system-scope stores, store_shared), so no L2 writeback of the
// whole cache is needed; it waits for them, then adds, also at system scope.
// Consumers poll the counters with loads that bypass the caches (lane l of
// wave 0 reads counter l).  A consumer that reads the results only with
// load_shared4 needs nothing more; one that reads them with ordinary loads
// invalidates its caches first (agent-scope acquire).  ctr[0] counts the
// tickets consumers took after their wait; ctr[2] is set if a wait gave up
// (read by dbf_workspace_check).
struct Sync {
  unsigned* ctr;
  unsigned* slots;
  unsigned n_prod, n_cons;
};

inline Sync make_sync(void* ws, int64_t n_prod, int64_t n_cons) {
  Sync s;
  s.ctr = static_cast<unsigned*>(ws);
  s.slots = reinterpret_cast<unsigned*>(static_cast<unsigned char*>(ws) + 256);
  s.n_prod = static_cast<unsigned>(n_prod);
  s.n_cons = static_cast<unsigned>(n_cons);
  return s;
}

// Producer `pid`, called by all threads after its store_shared results:
// the storing wave (wave 0) waits for their completion, then adds.
__device__ __forceinline__ void publish(const Sync& s, unsigned pid) {
  if (threadIdx.x == 0) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are complete
    __hip_atomic_fetch_add(s.slots + (pid % kSyncSlots) * kSyncStride, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// Consumer: lane l of wave 0 polls counter l until every counter holds its
// count, then acquires (an agent-scope invalidation of L1 and L2, about a
// microsecond; a consumer that reads the results only with load_shared4
// passes acquire = false); the workgroup barrier orders the other waves
// after it.
__device__ __forceinline__ void wait_producers(const Sync& s, bool acquire = true) {
  static_assert(kSyncSlots <= 64, "one counter per lane");
  if (threadIdx.x < 64) {
    const unsigned lane = threadIdx.x;
    const unsigned ns = static_cast<unsigned>(kSyncSlots);
    const unsigned want = lane < ns ? s.n_prod / ns + (lane < s.n_prod % ns ? 1u : 0u) : 0u;
    unsigned spins = 0;
    while (true) {
      const unsigned have =
          want > 0u ? __hip_atomic_load(s.slots + lane * kSyncStride, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_SYSTEM)
                    : 0u;
      if (__all(have >= want)) break;
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        if (lane == 0)
          __hip_atomic_fetch_or(s.ctr + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        break;
      }
    }
    if (acquire) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  // loads issued before the wait (prefetched inputs) are complete by now;
  // waiting for them here costs nothing and lets the compiler's later waits
  // count only loads issued after this point
  __builtin_amdgcn_s_waitcnt(0);
}

// Consumer, once past wait_producers: thread 0 takes a ticket (the order in
// which consumers got here), which only consumer_done reads.  A wave's loads
// return in order, so a consumer takes it after issuing its first loads of
// the producers' results; its round trip then overlaps the work on them.
__device__ __forceinline__ unsigned take_ticket(const Sync& s) {
  unsigned ticket = 0;
  if (threadIdx.x == 0)
    ticket = __hip_atomic_fetch_add(s.ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  return ticket;
}

// The same ticket, taken by the calling lane (one lane of any wave).
__device__ __forceinline__ unsigned take_ticket_any(const Sync& s) {
  return __hip_atomic_fetch_add(s.ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Consumer, at its end, with its ticket: the last consumer to take one
// (every producer has published and every consumer has passed its wait by
// then) clears the counters for the next call.
__device__ __forceinline__ void consumer_done(const Sync& s, unsigned ticket) {
  if (threadIdx.x < 64) {
    // thread 0 holds the ticket; the lanes of wave 0 clear one counter each
    if (__builtin_amdgcn_readfirstlane(ticket) == s.n_cons - 1u) {
      if (threadIdx.x < kSyncSlots)
        __hip_atomic_store(s.slots + threadIdx.x * kSyncStride, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
      if (threadIdx.x == 0) __hip_atomic_store(s.ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

// ---- several adapters, one per token (multi-adapter serving) ------------
// The adapter table travels in the kernel arguments.  token_adapter reads a
// token's adapter index; an index outside [-1, n) is taken as -1 (no
// adapter) and raises flag ctr[3] of the workspace head.
struct AdapterTable {
  const uint32_t* b1[kMaxAdapters];
  const uint32_t* b2[kMaxAdapters];
  const uint16_t* alpha[kMaxAdapters];
  const uint16_t* beta[kMaxAdapters];
  const uint16_t* gamma[kMaxAdapters];
  int n;
};

__device__ __forceinline__ int token_adapter(const int32_t* idx, int64_t tok,
                                             const AdapterTable& tab, const Sync& sync,
                                             bool flag) {
  const int a = idx[tok];
  if (a < -1 || a >= tab.n) {
    if (flag && threadIdx.x == 0)
      __hip_atomic_fetch_or(sync.ctr + 3, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    return -1;
  }
  return a;
}

// Splits of stage 1 along M (at most kMaxKS, each a whole number of passes'
// worth of nw K-blocks) so that stage 1 has about `want_wg` workgroups of nw
// waves.
inline int pick_ks(int64_t nrt, int n_terms, int64_t nkb, int64_t want_wg,
                   int64_t* kb_per_split, int nw = kWaves) {
  const int64_t want = want_wg / std::max<int64_t>(1, nrt * n_terms);
  const int64_t maxks = std::max<int64_t>(1, nkb / nw);
  int64_t ks = std::max<int64_t>(1, std::min<int64_t>(std::min(want, maxks), kMaxKS));
  int64_t per = (nkb + ks - 1) / ks;
  per = (per + nw - 1) / nw * nw;
  ks = (nkb + per - 1) / per;
  *kb_per_split = per;
  return static_cast<int>(ks);
}

}  // namespace lut

// Stage-1 parameters of the decode path for these sizes and workgroups of
// nw waves (K-split so that stage 1 has enough waves when `split`, else as
// few splits as the partial buffer allows); *n1 = its number of workgroups.
// ws is the caller's workspace (counters first).
lut::Stage1 make_stage1(const TermPtrs& t, int64_t M, int64_t R, const void* x,
                        int x_dtype, int64_t T, int64_t ldx, void* ws, bool split,
                        int* n1, int nw = lut::kWaves);

}  // namespace dbf
