// Quantized MoE dispatch: FP8 e4m3 payload with one fp32 scale per group.
//
// "集合通信：原语、算法、NCCL 实现与拓扑映射" (hpc/04), section 4.3: the
// dispatch direction of an MoE layer may travel as FP8 e4m3 while the
// combine direction stays bf16, which halves the dispatch bytes.  The
// format is the OCP E4M3 one (bias 7, subnormals m * 2^-9, no infinities,
// S.1111.111 = NaN, largest finite 448).
//
// Pack: one wave per (rank, token).  The token row is loaded once into
// registers (16 elements = two 16-byte vectors per unit, units j =
// u*64 + lane), every group's amax is reduced with lane shuffles (groups
// of up to 1024 elements sit inside one unit column of the wave; larger
// groups span whole unit columns), each element is multiplied by
// 448/amax and encoded, and the codes, scales and padding are written to
// the packed row of every slot (assignment) of the token.
//
// Encoding and decoding use the gfx950 FP8 conversion instructions, which
// implement OCP E4M3 with round to nearest even; magnitudes are clamped to
// 448 before encoding (the format's saturating reading).  Their results
// were compared with the format's definition for every fp32 bit pattern
// up to infinity (encode) and every code (decode).
//
// Dequant: one wave per received row; codes decode exactly to fp32, are
// multiplied by the group scale and narrowed to bf16 (round to nearest
// even).  Rows per rank come from the byte counts on the device.
#include "device_common.h"
#include "moe_direct.h"

namespace coll {

namespace {

constexpr int kLanes = 64;

__device__ __forceinline__ uint64_t fp8_wave_id() {
  return (uint64_t)blockIdx.x * (kBlock / kLanes) + (uint64_t)__builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
}
__device__ __forceinline__ uint64_t fp8_wave_count() { return (uint64_t)gridDim.x * (kBlock / kLanes); }

// Four e4m3 codes (bytes 0..3) of four fp32 values: round to nearest
// even through the gfx950 conversion instruction (v_cvt_pk_fp8_f32, OCP
// E4M3), after clamping to +-448 so that larger magnitudes saturate
// instead of becoming NaN.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
  d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Largest |x| of 16 bf16 elements, as a bf16 pattern: for finite values
// the magnitude order is the integer order of the low 15 bits, so the two
// halves of every word are compared with one packed 16-bit max.
__device__ __forceinline__ uint32_t unit_amax_bits(const u32x4& x0, const u32x4& x1) {
  u16x2 m = {0, 0};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, x0[e] & 0x7fff7fffu));
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, x1[e] & 0x7fff7fffu));
  }
  return m[0] > m[1] ? m[0] : m[1];
}

// Codes of 16 bf16 elements (x0: elements 0..7, x1: 8..15) times inv.
__device__ __forceinline__ u32x4 unit_codes(const u32x4& x0, const u32x4& x1, float inv) {
  u32x4 out;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4& x = q < 2 ? x0 : x1;
    const uint32_t w0 = x[2 * (q & 1)], w1 = x[2 * (q & 1) + 1];
    out[q] = e4m3_pack4(bf16_lo(w0) * inv, bf16_hi(w0) * inv, bf16_lo(w1) * inv, bf16_hi(w1) * inv);
  }
  return out;
}

}  // namespace

// Where the encoded slot rows of a token go.  Rows<Fp8Args>: the rank's
// packed buffer, row = pos (coll_moe_pack_fp8).  Rows<MoeDirectArgs>: the
// destination's receive buffer at the placement-table row, with the
// location written back once the token is done (coll_moe_dispatch_fp8).
template <class Args> struct Rows;

template <> struct Rows<Fp8Args> {
  const Fp8Args& a;
  __device__ uint8_t* slot_row(int rank, uint64_t x, int64_t& loc) const {
    loc = -1;
    const int32_t ps = as_global(a.pos[rank])[x];
    if (ps < 0 || (uint64_t)ps >= a.tokens * (uint64_t)a.k) return nullptr;
    return as_global((uint8_t*)a.dst[rank]) + (uint64_t)ps * a.row_bytes;
  }
  __device__ void finish(int, uint64_t, const int64_t (&)[kMaxTopK], int) const {}
};

template <> struct Rows<MoeDirectArgs> {
  const MoeDirectArgs& a;
  const int32_t* soff;
  const int32_t* roff;
  bool reject;
  __device__ uint8_t* slot_row(int rank, uint64_t x, int64_t& loc) const {
    loc = -1;
    if (reject) return nullptr;
    // every lane reads the same words: keep them in scalar registers
    const int32_t ps = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(uint64_t)as_global(a.loc[rank])[x]);
    if (ps < 0 || (uint64_t)ps >= a.tokens * (uint64_t)a.k) return nullptr;
    const int j = __builtin_amdgcn_readfirstlane(as_global(a.dest[rank])[x]);
    if (j < 0 || j >= a.p) return nullptr;
    const int64_t row = (int64_t)roff[rank * a.p + j] + (ps - soff[rank * a.p + j]);
    loc = direct_loc(j, row);
    return as_global((uint8_t*)a.dst[j]) + (uint64_t)row * a.row_bytes;
  }
  // after every read of the token's locations
  __device__ void finish(int rank, uint64_t x0, const int64_t (&loc)[kMaxTopK], int lane) const {
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s)
      if (s < a.k && lane == 0) as_global(a.loc[rank])[x0 + s] = loc[s];
  }
};

__device__ __forceinline__ Rows<Fp8Args> make_rows(const Fp8Args& a, int32_t*, int*) { return Rows<Fp8Args>{a}; }
__device__ __forceinline__ Rows<MoeDirectArgs> make_rows(const MoeDirectArgs& a, int32_t* tabs, int* flag) {
  const bool reject = direct_tables(a, tabs, tabs + a.p * a.p, flag);
  return Rows<MoeDirectArgs>{a, tabs, tabs + a.p * a.p, reject};
}

// The destination rows of token t's k slots (nullptr: not delivered).
template <class Args>
__device__ __forceinline__ bool slot_rows(const Rows<Args>& tgt, const Args& a, int rank, uint64_t t,
                                          uint8_t* (&row)[kMaxTopK], int64_t (&loc)[kMaxTopK]) {
  bool any = false;
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s) {
    row[s] = nullptr;
    loc[s] = -1;
    if (s < a.k) {
      row[s] = tgt.slot_row(rank, t * (uint64_t)a.k + s, loc[s]);
      any |= row[s] != nullptr;
    }
  }
  return any;
}

// Groups of at most 1024 elements (g16 <= 64 units): every group lies in
// one unit column (64 adjacent units), so a row streams through in
// batches of CB columns and any hidden size works.
//
// A wave walks its (row, batch) steps with the next step's loads issued
// before the current step's amax, encoding and stores, so the token reads
// of one row overlap the code writes of the previous one (gfx9 counts
// loads and stores on one counter: loads issued after a store would wait
// for it).  Rows whose slots are all undelivered load nothing.
constexpr int kPackCols = 8;

template <int CB, class Args>
COLL_STREAM_KERNEL void moe_pack_fp8_cols_kernel(Args a) {
#pragma clang fp contract(off)
  extern __shared__ int32_t tabs[];  // direct dispatch: placement tables
  __shared__ int flag;
  const Rows<Args> tgt = make_rows(a, tabs, &flag);
  const int lane = (int)(threadIdx.x % kLanes);
  const uint64_t H = a.hidden;
  const uint32_t nunits = (uint32_t)(H / 16);
  const uint32_t ncols = (nunits + kLanes - 1) / kLanes;
  const uint32_t g16 = (uint32_t)(a.group / 16);          // a power of two <= 64
  const uint32_t gsh = 31u - (uint32_t)__builtin_clz(g16);
  const uint32_t ngroups = (uint32_t)(H / a.group);
  const uint32_t npad = (uint32_t)((a.row_bytes - H) / 4) - ngroups;
  const uint64_t rows = a.tokens * (uint64_t)a.p;
  const uint64_t waves = fp8_wave_count();

  // the row of step (r, c0): its source and slot destinations
  struct RowState {
    uint64_t r;
    int rank;
    uint64_t t;
    bool any;
    const u32x4* src;
    uint8_t* drow[kMaxTopK];
    int64_t loc[kMaxTopK];
  };
  auto open_row = [&](uint64_t r, RowState& st) {
    st.r = r;
    st.rank = (int)(r / a.tokens);
    st.t = r - (uint64_t)st.rank * a.tokens;
    st.any = slot_rows(tgt, a, st.rank, st.t, st.drow, st.loc);
    st.src = reinterpret_cast<const u32x4*>(as_global((const uint16_t*)a.src[st.rank]) + st.t * H);
  };
  auto load = [&](const RowState& st, uint32_t c0, u32x4 (&x)[CB][2]) {
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const uint32_t j = (c0 + u) * kLanes + lane;
      if (st.any && j < nunits) {
        x[u][0] = ld16<true>(st.src + 2 * j);
        x[u][1] = ld16<true>(st.src + 2 * j + 1);
      } else {
        x[u][0] = u32x4{0, 0, 0, 0};
        x[u][1] = u32x4{0, 0, 0, 0};
      }
    }
  };

  uint64_t r = fp8_wave_id();
  if (r >= rows) return;
  RowState cur, nxt;
  open_row(r, cur);
  uint32_t c0 = 0;
  u32x4 x[CB][2];
  load(cur, c0, x);
  while (true) {
    // the next step: the next batch of this row, or the wave's next row
    const bool row_done = c0 + CB >= ncols;
    const uint32_t cn = row_done ? 0u : c0 + CB;
    const bool more = !row_done || cur.r + waves < rows;
    if (row_done && more) open_row(cur.r + waves, nxt);
    u32x4 xn[CB][2];
    if (more) load(row_done ? nxt : cur, cn, xn);
    if (cur.any) {
      uint32_t mb[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        mb[u] = unit_amax_bits(x[u][0], x[u][1]);
        for (uint32_t off = 1; off < g16; off <<= 1) mb[u] = max(mb[u], (uint32_t)__shfl_xor((int)mb[u], (int)off));
      }
      float sc[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const float amax = fmaxf(__uint_as_float(mb[u] << 16), 0x1p-110f);
        x[u][0] = unit_codes(x[u][0], x[u][1], 448.0f / amax);
        sc[u] = amax / 448.0f;
      }
#pragma unroll
      for (int s = 0; s < kMaxTopK; ++s) {
        if (!cur.drow[s]) continue;
        u32x4* vc = as_global(reinterpret_cast<u32x4*>(cur.drow[s]));
        float* scales = as_global(reinterpret_cast<float*>(cur.drow[s] + H));
#pragma unroll
        for (int u = 0; u < CB; ++u) {
          const uint32_t j = (c0 + u) * kLanes + lane;
          if (j < nunits) {
            st16<true>(vc + j, x[u][0]);
            if ((j & (g16 - 1)) == 0) scales[j >> gsh] = sc[u];
          }
        }
        if (row_done && (uint32_t)lane < npad) scales[ngroups + lane] = 0.0f;
      }
    }
    if (row_done) tgt.finish(cur.rank, cur.t * (uint64_t)a.k, cur.loc, lane);
    if (!more) break;
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      x[u][0] = xn[u][0];
      x[u][1] = xn[u][1];
    }
    if (row_done) cur = nxt;
    c0 = cn;
  }
}

// Groups spanning whole unit columns (group a multiple of 1024): the row
// is held in registers, UMAX units per lane (a power of two, hidden <=
// 64 * 16 * UMAX), and a group's amax is reduced over the wave and over
// its gu columns before any code is written.
template <int UMAX, class Args>
COLL_STREAM_KERNEL void moe_pack_fp8_rows_kernel(Args a) {
#pragma clang fp contract(off)
  extern __shared__ int32_t tabs[];
  __shared__ int flag;
  const Rows<Args> tgt = make_rows(a, tabs, &flag);
  const int lane = (int)(threadIdx.x % kLanes);
  const uint64_t H = a.hidden;
  const uint32_t nunits = (uint32_t)(H / 16);
  const uint32_t g16 = (uint32_t)(a.group / 16);
  const uint32_t gu = g16 / kLanes;                       // unit columns per group
  const uint32_t ngroups = (uint32_t)(H / a.group);
  const uint32_t npad = (uint32_t)((a.row_bytes - H) / 4) - ngroups;
  const uint64_t rows = a.tokens * (uint64_t)a.p;
  for (uint64_t r = fp8_wave_id(); r < rows; r += fp8_wave_count()) {
    const int rank = (int)(r / a.tokens);
    const uint64_t t = r - (uint64_t)rank * a.tokens;
    uint8_t* drow[kMaxTopK];
    int64_t loc[kMaxTopK];
    if (slot_rows(tgt, a, rank, t, drow, loc)) {
      const u32x4* src = reinterpret_cast<const u32x4*>(as_global((const uint16_t*)a.src[rank]) + t * H);
      u32x4 x[UMAX][2];
#pragma unroll
      for (int u = 0; u < UMAX; ++u) {
        const uint32_t j = (uint32_t)(u * kLanes + lane);
        if (j < nunits) {
          x[u][0] = ld16<true>(src + 2 * j);
          x[u][1] = ld16<true>(src + 2 * j + 1);
        } else {
          x[u][0] = u32x4{0, 0, 0, 0};
          x[u][1] = u32x4{0, 0, 0, 0};
        }
      }
      uint32_t mb[UMAX];
#pragma unroll
      for (int u = 0; u < UMAX; ++u) {
        mb[u] = unit_amax_bits(x[u][0], x[u][1]);
#pragma unroll
        for (int off = 1; off < kLanes; off <<= 1) mb[u] = max(mb[u], (uint32_t)__shfl_xor((int)mb[u], off));
      }
      uint32_t gm[UMAX];  // amax of the unit's group (all its columns)
#pragma unroll
      for (int u = 0; u < UMAX; ++u) {
        const uint32_t gi = (uint32_t)u / gu;
        uint32_t m = 0;
#pragma unroll
        for (int v = 0; v < UMAX; ++v)
          if ((uint32_t)v / gu == gi) m = max(m, mb[v]);
        gm[u] = m;
      }
      float sc[UMAX];
#pragma unroll
      for (int u = 0; u < UMAX; ++u) {
        const float amax = fmaxf(__uint_as_float(gm[u] << 16), 0x1p-110f);
        sc[u] = amax / 448.0f;
        x[u][0] = unit_codes(x[u][0], x[u][1], 448.0f / amax);
      }
#pragma unroll
      for (int s = 0; s < kMaxTopK; ++s) {
        if (!drow[s]) continue;
        u32x4* vc = as_global(reinterpret_cast<u32x4*>(drow[s]));
        float* scales = as_global(reinterpret_cast<float*>(drow[s] + H));
#pragma unroll
        for (int u = 0; u < UMAX; ++u) {
          const uint32_t j = (uint32_t)(u * kLanes + lane);
          if (j < nunits) {
            st16<true>(vc + j, x[u][0]);
            if (lane == 0 && (uint32_t)u % gu == 0) scales[(uint32_t)u / gu] = sc[u];
          }
        }
        if ((uint32_t)lane < npad) scales[ngroups + lane] = 0.0f;
      }
    }
    tgt.finish(rank, t * (uint64_t)a.k, loc, lane);
  }
}

// out[rank] rows = dequantized received rows, in the order they arrived.
// Each lane takes units of 16 codes (one 16-byte load, 32 bytes of bf16
// out), DB units per lane per step.  In a step's batch of 64 units, lane
// 2m takes unit m and lane 2m + 1 unit 32 + m; neighbouring lanes swap
// one 16-byte half (DPP), so that lane L stores bytes 16L of the batch's
// first KiB and then 16L of its second: each store instruction writes
// 1 KiB contiguously.  With lane L storing both halves of unit L, each
// store instruction wrote every other 16 bytes of 2 KiB: 289-294 us
// against 264-267 us for the same bytes stored contiguously (4096 x 7168
// tokens, p = 8, top-2, G = 128).
constexpr int kDeqUnits = 4;

// v from the neighbouring lane (lanes 2m and 2m + 1 exchange).
__device__ __forceinline__ uint32_t swap_neighbour(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1 /* quad_perm 1,0,3,2 */, 0xF, 0xF, false);
}

template <int DB>
COLL_STREAM_KERNEL void moe_dequant_fp8_kernel(Fp8Args a) {
#pragma clang fp contract(off)
  __shared__ int64_t start[kMaxRanks + 1];
  __shared__ int bad;
  extern __shared__ int64_t cnt[];  // the p x p byte counts
  const int p = a.p;
  const int tid = threadIdx.x;
  const uint64_t H = a.hidden, R = a.row_bytes;
  if (tid == 0) bad = 0;
  // one load per thread, then the per-rank sums from LDS
  for (int x = tid; x < p * p; x += kBlock) cnt[x] = a.counts[x];
  __syncthreads();
  if (tid < p) {
    const int64_t cap = a.rows_cap[tid] * (int64_t)R;
    int64_t tot = 0;
    bool ok = true;
    for (int i = 0; i < p; ++i) {
      const int64_t c = cnt[i * p + tid];
      if (c < 0 || c > cap || c % (int64_t)R) ok = false;
      else tot += c;
    }
    if (tot > cap) ok = false;
    if (!ok) bad = 1;
    start[tid + 1] = tot / (int64_t)R;
  }
  __syncthreads();
  if (tid == 0) {
    start[0] = 0;
    for (int r = 0; r < p; ++r) start[r + 1] += start[r];
  }
  __syncthreads();
  const bool reject = bad != 0;
  if (blockIdx.x == 0 && tid == 0 && a.status) *a.status = reject ? 1 : 0;
  if (reject) return;
  const int lane = tid % kLanes;
  const uint32_t nunits = (uint32_t)(H / 16);
  // scale of unit j: j >> gsh for groups inside a unit column (a power of
  // two <= 64 units), else column / gu, the same for the whole wave
  const uint32_t g16 = (uint32_t)(a.group / 16);
  const bool in_col = g16 <= (uint32_t)kLanes;
  const uint32_t gsh = in_col ? 31u - (uint32_t)__builtin_clz(g16) : 0u;
  const uint32_t gu = in_col ? 1u : g16 / kLanes;
  const uint64_t total = (uint64_t)start[p];
  // A wave walks its (row, batch) steps with the next step's loads issued
  // before the current step's stores: loads and stores share one counter
  // on gfx9, so loads issued after a store would wait for it.
  auto row_of = [&](uint64_t g, const u32x4*& vc, const float*& sc, u32x4*& dst) {
    int rk = 0;
    while ((uint64_t)start[rk + 1] <= g) ++rk;
    const uint64_t row = g - (uint64_t)start[rk];
    const uint8_t* src = as_global((const uint8_t*)a.src[rk]) + row * R;
    vc = reinterpret_cast<const u32x4*>(src);
    sc = reinterpret_cast<const float*>(src + H);
    dst = reinterpret_cast<u32x4*>(as_global((uint16_t*)a.dst[rk]) + row * H);
  };
  // this lane's unit in a batch: m for lane 2m, 32 + m for lane 2m + 1
  const uint32_t mine = (uint32_t)(lane >> 1) + (uint32_t)(kLanes / 2) * (uint32_t)(lane & 1);
  auto load = [&](const u32x4* vc, const float* sc, uint32_t j0, u32x4 (&c)[DB], float (&s)[DB]) {
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const uint32_t j = j0 + b * kLanes + mine;
      c[b] = u32x4{0, 0, 0, 0};
      s[b] = 0.0f;
      if (j < nunits) {
        c[b] = ld16<true>(vc + j);
        s[b] = sc[in_col ? (j >> gsh) : (j0 / kLanes + b) / gu];
      }
    }
  };
  const uint64_t waves = fp8_wave_count();
  uint64_t g = fp8_wave_id();
  if (g >= total) return;
  uint32_t j0 = 0;
  const u32x4* vc;
  const float* sc;
  u32x4* dst;
  row_of(g, vc, sc, dst);
  u32x4 c[DB];
  float s[DB];
  load(vc, sc, j0, c, s);
  while (true) {
    uint64_t gn = g;
    uint32_t jn = j0 + DB * kLanes;
    if (jn >= nunits) {
      jn = 0;
      gn = g + waves;
    }
    const bool more = gn < total;
    const u32x4* vcn = vc;
    const float* scn = sc;
    u32x4* dstn = dst;
    if (more && gn != g) row_of(gn, vcn, scn, dstn);
    u32x4 cn[DB];
    float sn[DB];
    if (more) load(vcn, scn, jn, cn, sn);
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      // every lane converts (units past the row hold zero codes), so that
      // the exchange below reads active lanes only
      u32x4 y0, y1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // exact fp32 values of codes 0,1 and 2,3 of the word (v_cvt_pk_f32_fp8)
        const auto v01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[b][q], false);
        const auto v23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[b][q], true);
        u32x4& y = q < 2 ? y0 : y1;
        y[2 * (q & 1)] = bf16_pack(v01[0] * s[b], v01[1] * s[b]);
        y[2 * (q & 1) + 1] = bf16_pack(v23[0] * s[b], v23[1] * s[b]);
      }
      // lane 2m: its first half, then lane 2m + 1's first half; lane
      // 2m + 1: lane 2m's second half, then its own second half
      const bool odd = (lane & 1) != 0;
      u32x4 give = odd ? y0 : y1, got;
#pragma unroll
      for (int d = 0; d < 4; ++d) got[d] = swap_neighbour(give[d]);
      const u32x4 first = odd ? got : y0, second = odd ? y1 : got;
      const uint32_t jb = j0 + b * kLanes;  // the batch's first unit
      if (jb + (uint32_t)(lane >> 1) < nunits) st16<true>(dst + 2 * jb + lane, first);
      if (jb + (uint32_t)(kLanes / 2) + (uint32_t)(lane >> 1) < nunits)
        st16<true>(dst + 2 * jb + kLanes + lane, second);
    }
    if (!more) break;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      c[b] = cn[b];
      s[b] = sn[b];
    }
    g = gn;
    j0 = jn;
    vc = vcn;
    sc = scn;
    dst = dstn;
  }
}

template <class Args>
static int launch_pack_fp8_t(const Args& a, int max_grid, size_t shm, hipStream_t s) {
  const uint64_t rows = a.tokens * (uint64_t)a.p;
  const uint64_t wg_needed = (rows + (kBlock / kLanes) - 1) / (kBlock / kLanes);
  const int grid = (int)(wg_needed < (uint64_t)max_grid ? wg_needed : (uint64_t)max_grid);
  if (grid == 0) return 0;
  if (a.group <= 1024) {
    hipLaunchKernelGGL((moe_pack_fp8_cols_kernel<kPackCols, Args>), dim3(grid), dim3(kBlock), shm, s, a);
    return (int)hipGetLastError();
  }
  const uint64_t per_lane = (a.hidden / 16 + kLanes - 1) / kLanes;
  if (per_lane <= 1) hipLaunchKernelGGL((moe_pack_fp8_rows_kernel<1, Args>), dim3(grid), dim3(kBlock), shm, s, a);
  else if (per_lane <= 2) hipLaunchKernelGGL((moe_pack_fp8_rows_kernel<2, Args>), dim3(grid), dim3(kBlock), shm, s, a);
  else if (per_lane <= 4) hipLaunchKernelGGL((moe_pack_fp8_rows_kernel<4, Args>), dim3(grid), dim3(kBlock), shm, s, a);
  else if (per_lane <= 8) hipLaunchKernelGGL((moe_pack_fp8_rows_kernel<8, Args>), dim3(grid), dim3(kBlock), shm, s, a);
  else if (per_lane <= 16) hipLaunchKernelGGL((moe_pack_fp8_rows_kernel<16, Args>), dim3(grid), dim3(kBlock), shm, s, a);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int launch_moe_pack_fp8(const Fp8Args& a, int max_grid, void* stream) {
  return launch_pack_fp8_t(a, max_grid, 0, (hipStream_t)stream);
}

int launch_moe_dispatch_fp8(const MoeDirectArgs& a, int max_grid, void* stream) {
  return launch_pack_fp8_t(a, max_grid, direct_tables_bytes(a.p), (hipStream_t)stream);
}

int launch_moe_dequant_fp8(const Fp8Args& a, int max_grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const size_t shm = (size_t)a.p * a.p * sizeof(int64_t);
  hipLaunchKernelGGL((moe_dequant_fp8_kernel<kDeqUnits>), dim3(max_grid), dim3(kBlock), shm, s, a);
  return (int)hipGetLastError();
}

}  // namespace coll
