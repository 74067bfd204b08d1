// oracle.cpp - plain, slow CPU reference for the block-sparse mixed-precision
// (int8 / int4 / skip) causal attention path.
//
// TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check of __graft_entry__ and
// the cpu_baseline leg of bench.py may load this library.  It shares no code,
// header, table or constant with the GPU library: every layout and constant below
// is re-derived from the written contract and the pages it cites.
//
// Sources (cited by page and section):
//  * TriAttention summary page (rit.work, "TriAttention: sparse mixed-precision
//    attention"), section "which links can be skipped and which must not be
//    removed": three actions per tile (skip / 4 bits / 8 bits) chosen by distance
//    from the diagonal; the first key block and the diagonal block are always kept
//    at high precision; one pair of boundaries per head.
//  * same page, section "how calibration distributes compute between heads":
//    kept blocks are grouped by precision and reduced into one normalised result;
//    prepared keys and values go to a compressed KV cache read during generation.
//  * llmis.ru chapter 3.5 ("attention variants for inference"), section 2: the KV
//    cache byte formula 2*L*h*d_h*n*b*p; section 4: grouped-query attention.
//
// Readings taken where the pages are silent (each also listed in the design
// notes): boundaries inclusive and in blocks; per-row symmetric quantiser with
// qmax 127 / 7 and fp32 scales; both Q and K at 4 bits in an int4 tile; V in bf16
// for prefill; softmax weights rounded to bf16 after subtracting an integer
// maximum (power-of-two contract); cache and decode policies per KV head.
//
// Everything is double precision unless the contract fixes a narrower type.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// ---------------------------------------------------------------- bf16 / fp32
float bf16_to_float(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Round a finite float to bfloat16, nearest with ties to even (written out on the
// bit pattern: add half an ulp of the kept part, minus one when the kept lsb is 0).
uint16_t float_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return static_cast<uint16_t>(u >> 16);
}

// ---------------------------------------------------------------- tile actions
enum { ACT_NONCAUSAL = -1, ACT_SKIP = 0, ACT_INT4 = 4, ACT_INT8 = 8 };

// The distance-to-diagonal rule with the two protected blocks.
int tile_action(int64_t qb, int64_t kb, int64_t hi, int64_t keep) {
  if (kb > qb) return ACT_NONCAUSAL;
  int64_t dist = qb - kb;
  if (kb == 0 || dist == 0) return ACT_INT8;  // protected: first key block, diagonal
  if (dist <= hi) return ACT_INT8;
  if (dist <= keep) return ACT_INT4;
  return ACT_SKIP;
}

// ---------------------------------------------------------------- quantiser
// Symmetric per-row quantiser: scale = amax/qmax, code = clamp(rint(x*(qmax/amax))).
void quantize_row(const uint16_t* x, int d, int qmax, int8_t* codes, float* scale) {
  float amax = 0.0f;
  for (int i = 0; i < d; ++i) amax = std::max(amax, std::fabs(bf16_to_float(x[i])));
  if (amax == 0.0f) {
    *scale = 0.0f;
    for (int i = 0; i < d; ++i) codes[i] = 0;
    return;
  }
  const float fq = static_cast<float>(qmax);
  *scale = amax / fq;
  const float r = fq / amax;
  for (int i = 0; i < d; ++i) {
    float c = std::rint(bf16_to_float(x[i]) * r);
    c = std::min(std::max(c, -fq), fq);
    codes[i] = static_cast<int8_t>(c);
  }
}

uint8_t pack_pair(int8_t even, int8_t odd) {
  return static_cast<uint8_t>((static_cast<uint8_t>(even) & 0x0Fu) |
                              ((static_cast<uint8_t>(odd) & 0x0Fu) << 4));
}

// ---------------------------------------------------------------- threading
template <class F>
void parallel_for(int64_t count, int nthreads, F fn) {
  if (nthreads < 1) nthreads = 1;
  std::atomic<int64_t> next{0};
  auto worker = [&]() {
    for (;;) {
      int64_t i = next.fetch_add(1);
      if (i >= count) break;
      fn(i);
    }
  };
  std::vector<std::thread> pool;
  for (int t = 1; t < nthreads; ++t) pool.emplace_back(worker);
  worker();
  for (auto& th : pool) th.join();
}

struct QuantRows {  // codes and scales of a set of rows at one precision
  std::vector<int8_t> codes;
  std::vector<float> scales;
};

QuantRows quantize_all(const uint16_t* x, int64_t rows, int d, int qmax, int nthreads) {
  QuantRows r;
  r.codes.resize(static_cast<size_t>(rows) * d);
  r.scales.resize(static_cast<size_t>(rows));
  parallel_for((rows + 1023) / 1024, nthreads, [&](int64_t c) {
    for (int64_t i = c * 1024; i < std::min(rows, (c + 1) * 1024); ++i)
      quantize_row(x + i * d, d, qmax, &r.codes[i * d], &r.scales[i]);
  });
  return r;
}

// Per-KV-head boundaries: either given per KV head, or merged from per-query-head
// values by the group maximum (the union of what the group's heads keep).
void kv_policy(int n_q_heads, int n_kv_heads, const int32_t* hi, const int32_t* keep,
               int n_policy_heads, std::vector<int64_t>& hk, std::vector<int64_t>& kk) {
  hk.assign(n_kv_heads, 0);
  kk.assign(n_kv_heads, 0);
  if (n_policy_heads == n_kv_heads) {
    for (int g = 0; g < n_kv_heads; ++g) { hk[g] = hi[g]; kk[g] = keep[g]; }
    return;
  }
  const int G = n_q_heads / n_kv_heads;
  for (int h = 0; h < n_q_heads; ++h) {
    hk[h / G] = std::max<int64_t>(hk[h / G], hi[h]);
    kk[h / G] = std::max<int64_t>(kk[h / G], keep[h]);
  }
}

void put_i32(uint8_t* dst, int32_t v) { std::memcpy(dst, &v, 4); }
void put_i64(uint8_t* dst, int64_t v) { std::memcpy(dst, &v, 8); }
void put_f32(uint8_t* dst, float v) { std::memcpy(dst, &v, 4); }

// Token of position p (0..31) of a 32-token chunk in the transposed V codes
// (the documented feed order of the cache): position 8q + p' holds token
// 16(p' / 4) + 4q + p' % 4.
int feed_token(int pos) {
  int q = pos / 8, p = pos % 8;
  return 16 * (p / 4) + 4 * q + (p % 4);
}

// One stored block as the cache's record: 32-token chunks, each holding a K part,
// a V part and the chunk's scales, the parts being sequences of 16-byte units
// (one per lane of a 1 KB load; lane = r + 16q):
//   int8 K: unit (s, ks, q, r) = dims 64ks+16q .. +15 of token 32c+16s+r
//   int4 K: unit (s, q, r)     = for ks = 0..d/64-1, dims 64ks+16q .. +15 packed into
//                                8 bytes (low nibble = even dim)   [8*(d/64) bytes]
//   int8 V: unit (m, q, r)     = for dt = 2m, 2m+1: 8 bytes, position p = dim 16dt+r of
//                                token 32c + 16(p/4) + 4q + p%4
//   int4 V: unit (m, q, r)     = for dt = 4m..4m+3: those 8 positions packed into 4
//                                bytes (low nibble = even p)
//   then K scales fp32 [32] and V scales fp32 [32].
// This is the order in which one decode step of 32 tokens consumes them.
void write_record(const int8_t* kc, const int8_t* vc, const float* ks, const float* vs, int block, int d,
                  bool int4, uint8_t* rec) {
  const int ksl = d / 64;
  const int64_t part = int4 ? 16LL * d : 32LL * d;  // bytes of the K (and of the V) part of a chunk
  for (int c = 0; c < block / 32; ++c) {
    uint8_t* ck = rec + c * (2 * part + 256);
    uint8_t* cv = ck + part;
    uint8_t* cs = cv + part;
    // K part
    int64_t o = 0;
    if (!int4) {
      for (int s = 0; s < 2; ++s)
        for (int kk = 0; kk < ksl; ++kk)
          for (int q = 0; q < 4; ++q)
            for (int r = 0; r < 16; ++r) {
              const int8_t* row = kc + static_cast<size_t>(32 * c + 16 * s + r) * d + 64 * kk + 16 * q;
              for (int i = 0; i < 16; ++i) ck[o++] = static_cast<uint8_t>(row[i]);
            }
    } else {
      for (int s = 0; s < 2; ++s)
        for (int q = 0; q < 4; ++q)
          for (int r = 0; r < 16; ++r)
            for (int kk = 0; kk < ksl; ++kk) {
              const int8_t* row = kc + static_cast<size_t>(32 * c + 16 * s + r) * d + 64 * kk + 16 * q;
              for (int i = 0; i < 16; i += 2) ck[o++] = pack_pair(row[i], row[i + 1]);
            }
    }
    // V part
    o = 0;
    const int per = int4 ? 4 : 2;  // dim groups per unit
    for (int m = 0; m < d / 16 / per; ++m)
      for (int q = 0; q < 4; ++q)
        for (int r = 0; r < 16; ++r)
          for (int t = 0; t < per; ++t) {
            const int dim = 16 * (per * m + t) + r;
            for (int p = 0; p < 8; ++p) {
              const int8_t x = vc[static_cast<size_t>(32 * c + feed_token(8 * q + p)) * d + dim];
              if (!int4) {
                cv[o++] = static_cast<uint8_t>(x);
              } else if (p % 2 == 0) {
                const int8_t y = vc[static_cast<size_t>(32 * c + feed_token(8 * q + p + 1)) * d + dim];
                cv[o++] = pack_pair(x, y);
              }
            }
          }
    for (int t = 0; t < 32; ++t) {
      put_f32(cs + 4 * t, ks[32 * c + t]);
      put_f32(cs + 128 + 4 * t, vs[32 * c + t]);
    }
  }
}

}  // namespace

extern "C" {

// ============================================================ pins and helpers
// The pages' KV-cache formula (llmis.ru chapter 3.5, section 2): keys and values
// of L layers, h heads of size d_h, n tokens, batch b, p bytes per element.
int64_t oracle_kv_formula_bytes(int64_t L, int64_t h, int64_t d_h, int64_t n, int64_t b, int64_t p) {
  return 2 * L * h * d_h * n * b * p;
}

int oracle_tile_action(int64_t qb, int64_t kb, int64_t hi, int64_t keep) {
  return tile_action(qb, kb, hi, keep);
}

float oracle_bf16_to_float(uint16_t b) { return bf16_to_float(b); }
uint16_t oracle_float_to_bf16(float f) { return float_to_bf16(f); }

void oracle_quantize_rows(const uint16_t* x, int64_t rows, int d, int qmax, int8_t* codes,
                          float* scales) {
  for (int64_t i = 0; i < rows; ++i) quantize_row(x + i * d, d, qmax, codes + i * d, scales + i);
}

void oracle_pack_nibbles(const int8_t* codes, int64_t count, uint8_t* out) {
  for (int64_t j = 0; j < count / 2; ++j) out[j] = pack_pair(codes[2 * j], codes[2 * j + 1]);
}

// Dense softmax attention in double, with an arbitrary key mask (1 = keep):
// out_i = sum_j mask_ij exp(scale q_i.k_j) v_j / sum_j mask_ij exp(scale q_i.k_j).
// q, k have dk columns and v, out have dv.  Rows with no kept key get zeros.
void oracle_dense_attention(const double* q, const double* k, const double* v, int64_t nq,
                            int64_t nk, int dk, int dv, const uint8_t* mask, double scale,
                            double* out) {
  std::vector<double> s(static_cast<size_t>(nk));
  for (int64_t i = 0; i < nq; ++i) {
    double mx = -INFINITY;
    for (int64_t j = 0; j < nk; ++j) {
      if (!mask[i * nk + j]) continue;
      double acc = 0.0;
      for (int c = 0; c < dk; ++c) acc += q[i * dk + c] * k[j * dk + c];
      s[j] = scale * acc;
      mx = std::max(mx, s[j]);
    }
    double den = 0.0;
    for (int c = 0; c < dv; ++c) out[i * dv + c] = 0.0;
    if (mx == -INFINITY) continue;
    for (int64_t j = 0; j < nk; ++j) {
      if (!mask[i * nk + j]) continue;
      double p = std::exp(s[j] - mx);
      den += p;
      for (int c = 0; c < dv; ++c) out[i * dv + c] += p * v[j * dv + c];
    }
    for (int c = 0; c < dv; ++c) out[i * dv + c] /= den;
  }
}

// ============================================================ (1) schedule
int64_t oracle_schedule_bytes(int64_t batch, int64_t n_q_heads, int64_t nb) {
  return 64 + 32 * batch * n_q_heads * nb;
}

// Builds the canonical schedule from the per-tile action map: for each unit the
// int8 run that ends at the diagonal, the int4 blocks, and block 0 when it is
// int8 but not part of the run.  Returns 0, or -1 if the action map is not of
// the documented shape (which would mean the rule itself is broken).
int oracle_build_schedule(int batch, int n_q_heads, int n_kv_heads, int head_dim, int block,
                          int64_t seq_len, const int32_t* hi, const int32_t* keep,
                          int32_t* out, int64_t out_words) {
  const int64_t nb = (seq_len + block - 1) / block;
  const int64_t n_units = static_cast<int64_t>(batch) * n_q_heads * nb;
  if (out_words < 16 + 8 * n_units) return -1;
  struct Unit { int32_t f[8]; };
  std::vector<Unit> units;
  units.reserve(static_cast<size_t>(n_units));
  for (int b = 0; b < batch; ++b)
    for (int h = 0; h < n_q_heads; ++h)
      for (int64_t qb = 0; qb < nb; ++qb) {
        std::vector<int> act(static_cast<size_t>(qb + 1));
        for (int64_t kb = 0; kb <= qb; ++kb) act[kb] = tile_action(qb, kb, hi[h], keep[h]);
        int64_t lo8 = qb;
        while (lo8 > 0 && act[lo8 - 1] == ACT_INT8) --lo8;
        // block 0 is int8 by protection; if the run stops above it, it is the sink
        int32_t sink = (lo8 > 0 && act[0] == ACT_INT8) ? 1 : 0;
        int64_t lo4 = -1, hi4 = -1, n4 = 0, kept = 0;
        for (int64_t kb = 0; kb <= qb; ++kb) {
          if (act[kb] != ACT_SKIP) ++kept;
          if (act[kb] == ACT_INT4) {
            if (lo4 < 0) lo4 = kb;
            hi4 = kb;
            ++n4;
          }
        }
        if (n4 == 0) { lo4 = 0; hi4 = -1; }
        if (n4 != hi4 - lo4 + 1 && n4 != 0) return -1;          // int4 blocks not contiguous
        if (kept != (qb - lo8 + 1) + sink + n4) return -1;      // int8 blocks not {0} u run
        Unit u;
        int32_t f[8] = {b, h, static_cast<int32_t>(qb), static_cast<int32_t>(lo8),
                        static_cast<int32_t>(lo4), static_cast<int32_t>(hi4), sink,
                        static_cast<int32_t>(kept)};
        std::memcpy(u.f, f, sizeof f);
        units.push_back(u);
      }
  std::stable_sort(units.begin(), units.end(), [](const Unit& a, const Unit& b) {
    if (a.f[7] != b.f[7]) return a.f[7] > b.f[7];
    if (a.f[0] != b.f[0]) return a.f[0] < b.f[0];
    if (a.f[1] != b.f[1]) return a.f[1] < b.f[1];
    return a.f[2] < b.f[2];
  });
  std::memset(out, 0, sizeof(int32_t) * 16);
  out[0] = 0x48435354;  // "TSCH"
  out[1] = 1;
  out[2] = batch; out[3] = n_q_heads; out[4] = n_kv_heads; out[5] = head_dim; out[6] = block;
  out[7] = static_cast<int32_t>(nb);
  out[8] = static_cast<int32_t>(n_units);
  out[10] = static_cast<int32_t>(seq_len & 0xFFFFFFFF);
  out[11] = static_cast<int32_t>(seq_len >> 32);
  for (int64_t i = 0; i < n_units; ++i) std::memcpy(out + 16 + 8 * i, units[i].f, 32);
  return 0;
}

// ============================================================ (3) prefill
// Follows the method row by row: keep the keys of non-skipped tiles, score them
// with the codes of the tile's precision, take an integer maximum, round the
// weights to bf16 and normalise by their sum.  `units` lists (b, h, qb) triples
// whose rows are computed (NULL with n_units = -1: all of them).  out and lse are
// full-size arrays; only the selected rows are written.  reference_mode = 1 keeps
// the weights in double (no bf16 rounding), for the exactness pins.
int oracle_prefill(int batch, int n_q_heads, int n_kv_heads, int d, int block, int64_t n,
                   const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* hi,
                   const int32_t* keep, float sm_scale, int reference_mode, const int32_t* units,
                   int64_t n_units, float* out, float* lse, int nthreads) {
  const int G = n_q_heads / n_kv_heads;
  const int64_t nb = (n + block - 1) / block;
  std::vector<int32_t> all;
  if (units == nullptr || n_units < 0) {
    for (int b = 0; b < batch; ++b)
      for (int h = 0; h < n_q_heads; ++h)
        for (int64_t qb = 0; qb < nb; ++qb) {
          all.push_back(b); all.push_back(h); all.push_back(static_cast<int32_t>(qb));
        }
    units = all.data();
    n_units = static_cast<int64_t>(all.size() / 3);
  }
  const int64_t k_rows = static_cast<int64_t>(batch) * n_kv_heads * n;
  QuantRows k8 = quantize_all(k, k_rows, d, 127, nthreads);
  QuantRows k4 = quantize_all(k, k_rows, d, 7, nthreads);
  const double log2e = 1.4426950408889634074;
  const double c = static_cast<double>(sm_scale) * log2e;

  parallel_for(n_units, nthreads, [&](int64_t u) {
    const int b = units[3 * u], h = units[3 * u + 1];
    const int64_t qb = units[3 * u + 2];
    const int g = h / G;
    const int64_t kbase = (static_cast<int64_t>(b) * n_kv_heads + g) * n;
    const int64_t qbase = (static_cast<int64_t>(b) * n_q_heads + h) * n;
    std::vector<int8_t> qc8(d), qc4(d);
    std::vector<double> t, w;
    std::vector<int64_t> keys;
    std::vector<double> o(d);
    for (int64_t i = qb * block; i < std::min(n, (qb + 1) * block); ++i) {
      float sq8, sq4;
      quantize_row(q + (qbase + i) * d, d, 127, qc8.data(), &sq8);
      quantize_row(q + (qbase + i) * d, d, 7, qc4.data(), &sq4);
      keys.clear();
      t.clear();
      for (int64_t j = 0; j <= i; ++j) {
        const int a = tile_action(qb, j / block, hi[h], keep[h]);
        if (a == ACT_SKIP) continue;
        const int8_t* qc = (a == ACT_INT8) ? qc8.data() : qc4.data();
        const int8_t* kc = (a == ACT_INT8) ? &k8.codes[(kbase + j) * d] : &k4.codes[(kbase + j) * d];
        int64_t s = 0;
        for (int x = 0; x < d; ++x) s += static_cast<int64_t>(qc[x]) * kc[x];
        const double sq = (a == ACT_INT8) ? sq8 : sq4;
        const double sk = (a == ACT_INT8) ? k8.scales[kbase + j] : k4.scales[kbase + j];
        keys.push_back(j);
        t.push_back(static_cast<double>(s) * sq * sk * c);
      }
      const double mx = *std::max_element(t.begin(), t.end());
      const double M = std::ceil(mx);
      w.resize(t.size());
      double l = 0.0;
      for (size_t x = 0; x < t.size(); ++x) {
        const double e = std::exp2(t[x] - M);
        if (reference_mode) {
          w[x] = e;
        } else {
          // fp32 first, then bf16; values below the normal fp32 range count as 0
          const float ef = static_cast<float>(e);
          w[x] = (ef < 0x1p-126f) ? 0.0 : static_cast<double>(bf16_to_float(float_to_bf16(ef)));
        }
        l += w[x];
      }
      std::fill(o.begin(), o.end(), 0.0);
      for (size_t x = 0; x < keys.size(); ++x) {
        const uint16_t* vr = v + (kbase + keys[x]) * d;
        for (int y = 0; y < d; ++y) o[y] += w[x] * static_cast<double>(bf16_to_float(vr[y]));
      }
      for (int y = 0; y < d; ++y) out[(qbase + i) * d + y] = static_cast<float>(o[y] / l);
      if (lse) lse[qbase + i] = static_cast<float>(M + std::log2(l));
    }
  });
  return 0;
}

// ============================================================ (4) cache
// Stored blocks of one KV head for query block c: the tile rule applied to the
// row of block c (int8 = protected blocks and the hi band, int4 = the keep band).
static void stored_sets(int64_t c, int64_t hi, int64_t keep, std::vector<int64_t>& b8,
                        std::vector<int64_t>& b4) {
  b8.clear();
  b4.clear();
  for (int64_t kb = 0; kb <= c; ++kb) {
    int a = tile_action(c, kb, hi, keep);
    if (a == ACT_INT8) b8.push_back(kb);
    if (a == ACT_INT4) b4.push_back(kb);
  }
}

// ============================================================ (f4) dynamic block skipping
// Source: rit.work page on ETA (Elastic Threshold Attention), section on how the
// model decides which part of the context to read: before a block is loaded, a few
// statistics of it (mean key, per-coordinate spread, largest key norm) give an upper
// bound on any of its scores; a block whose bound falls below the head's threshold
// is not read at all.  Same page: the whole cache stays stored, the statistics are
// a small extra index.
//
// Readings (also in the design notes): the statistics are taken over the stored
// codes of each stored block (all its rows; rows past ctx_len are zero), as
//   lo[x], hi[x]  per-coordinate minimum and maximum code  (mean +- spread, as a box)
//   smax          the largest row scale
//   nmax          the largest (sk * sk) * |kc|^2 over rows, in double
// For query head h (codes qc, scale sq at the block's precision) and a threshold
// theta in logit units (sm_scale * q.k), with t = sm_scale * sq (double):
//   box  = (t * smax) * max(sum_x max(qc_x lo_x, qc_x hi_x), 0)     >= any score
//   norm = ((t * t) * |qc|^2) * nmax                                 >= any score^2
// and the block is skipped for h iff theta > 0 and (box < theta or norm < theta^2).
// The first key block and the current block are never skipped (the blocks the tile
// rule always keeps).  A KV head's block is read if any of its query heads keeps it;
// each head attends over the blocks it keeps.
struct Summary {
  std::vector<int8_t> lo, hi;
  float smax = 0.0f;
  double nmax = 0.0;
};

static Summary summarise_block(const uint16_t* krows, int64_t first_tok, int64_t ctx_len, int block, int d, int qmax) {
  Summary s;
  s.lo.assign(d, 0);
  s.hi.assign(d, 0);
  std::vector<int8_t> kc(d);
  bool first = true;
  for (int r = 0; r < block; ++r) {
    float sk = 0.0f;
    std::fill(kc.begin(), kc.end(), 0);
    if (first_tok + r < ctx_len) quantize_row(krows + static_cast<int64_t>(r) * d, d, qmax, kc.data(), &sk);
    int64_t n2 = 0;
    for (int x = 0; x < d; ++x) {
      n2 += static_cast<int64_t>(kc[x]) * kc[x];
      s.lo[x] = first ? kc[x] : std::min(s.lo[x], kc[x]);
      s.hi[x] = first ? kc[x] : std::max(s.hi[x], kc[x]);
    }
    first = false;
    s.smax = std::max(s.smax, sk);
    s.nmax = std::max(s.nmax, (static_cast<double>(sk) * static_cast<double>(sk)) * static_cast<double>(n2));
  }
  return s;
}

// Stored blocks of KV head g in cache record order: int8 blocks ascending, then int4.
static void record_order(int64_t c, int64_t hi, int64_t keep, std::vector<int64_t>& blocks, std::vector<int>& qmaxs) {
  std::vector<int64_t> b8, b4;
  stored_sets(c, hi, keep, b8, b4);
  blocks = b8;
  blocks.insert(blocks.end(), b4.begin(), b4.end());
  qmaxs.assign(b8.size(), 127);
  qmaxs.insert(qmaxs.end(), b4.size(), 7);
}

static bool skip_for_head(const Summary& s, const int8_t* qc, float sq, float sm_scale, float theta, int d) {
  int64_t box = 0, q2 = 0;
  for (int x = 0; x < d; ++x) {
    box += std::max(static_cast<int64_t>(qc[x]) * s.lo[x], static_cast<int64_t>(qc[x]) * s.hi[x]);
    q2 += static_cast<int64_t>(qc[x]) * qc[x];
  }
  const double t = static_cast<double>(sm_scale) * static_cast<double>(sq);
  const double bound = (t * static_cast<double>(s.smax)) * static_cast<double>(std::max<int64_t>(box, 0));
  const double norm2 = ((t * t) * static_cast<double>(q2)) * s.nmax;
  const double th = theta;
  return th > 0.0 && (bound < th || norm2 < th * th);
}

// Keep masks of every stored record: bit i of masks[p * rmax + r] set = query head
// g*G + i keeps record r of pair p = b * n_kv_heads + g.  rmax = c + 1.
static void skip_masks(int batch, int n_q_heads, int n_kv_heads, int d, int block, int64_t n, int64_t ctx_len,
                       const std::vector<int64_t>& hk, const std::vector<int64_t>& kk, const uint16_t* k,
                       const uint16_t* q, const float* thresholds, float sm_scale, uint32_t* masks, int nthreads) {
  const int G = n_q_heads / n_kv_heads;
  const int64_t c = (ctx_len - 1) / block, rmax = c + 1;
  parallel_for(static_cast<int64_t>(batch) * n_kv_heads, nthreads, [&](int64_t p) {
    const int b = static_cast<int>(p / n_kv_heads), g = static_cast<int>(p % n_kv_heads);
    std::vector<int64_t> blocks;
    std::vector<int> qmaxs;
    record_order(c, hk[g], kk[g], blocks, qmaxs);
    std::vector<int8_t> qc8(static_cast<size_t>(G) * d), qc4(static_cast<size_t>(G) * d);
    std::vector<float> sq8(G), sq4(G);
    for (int i = 0; i < G; ++i) {
      const uint16_t* qr = q + (static_cast<int64_t>(b) * n_q_heads + g * G + i) * d;
      quantize_row(qr, d, 127, &qc8[static_cast<size_t>(i) * d], &sq8[i]);
      quantize_row(qr, d, 7, &qc4[static_cast<size_t>(i) * d], &sq4[i]);
    }
    const int64_t src = (static_cast<int64_t>(b) * n_kv_heads + g) * n;
    for (int64_t r = 0; r < rmax; ++r) masks[p * rmax + r] = 0;
    for (size_t r = 0; r < blocks.size(); ++r) {
      const int64_t kb = blocks[r];
      uint32_t m = 0;
      if (kb == 0 || kb == c) {
        m = G == 32 ? 0xFFFFFFFFu : ((1u << G) - 1u);
      } else {
        const Summary s = summarise_block(k + (src + kb * block) * d, kb * block, ctx_len, block, d, qmaxs[r]);
        for (int i = 0; i < G; ++i) {
          const bool is8 = qmaxs[r] == 127;
          const int8_t* qc = is8 ? &qc8[static_cast<size_t>(i) * d] : &qc4[static_cast<size_t>(i) * d];
          const float th = thresholds[static_cast<int64_t>(b) * n_q_heads + g * G + i];
          if (!skip_for_head(s, qc, is8 ? sq8[i] : sq4[i], sm_scale, th, d)) m |= 1u << i;
        }
      }
      masks[p * rmax + static_cast<int64_t>(r)] = m;
    }
  });
}

int64_t oracle_cache_bytes(int batch, int n_q_heads, int n_kv_heads, int d, int block,
                           int64_t ctx_len, const int32_t* hi, const int32_t* keep,
                           int n_policy_heads) {
  std::vector<int64_t> hk, kk, b8, b4;
  kv_policy(n_q_heads, n_kv_heads, hi, keep, n_policy_heads, hk, kk);
  const int64_t c = (ctx_len - 1) / block;
  int64_t total = 64 + 64 * static_cast<int64_t>(batch) * n_kv_heads;
  total = (total + 255) / 256 * 256;
  for (int b = 0; b < batch; ++b)
    for (int g = 0; g < n_kv_heads; ++g) {
      stored_sets(c, hk[g], kk[g], b8, b4);
      total += static_cast<int64_t>(b8.size()) * (2LL * block * d + 8LL * block) +
               static_cast<int64_t>(b4.size()) * (static_cast<int64_t>(block) * d + 8LL * block);
    }
  return total;
}

// Writes the documented cache bytes.  Returns 0, or -1 if out_bytes is too small.
int oracle_pack_cache(int batch, int n_q_heads, int n_kv_heads, int d, int block, int64_t n,
                      int64_t ctx_len, const int32_t* hi, const int32_t* keep, int n_policy_heads,
                      const uint16_t* k, const uint16_t* v, uint8_t* out, int64_t out_bytes) {
  const int64_t total = oracle_cache_bytes(batch, n_q_heads, n_kv_heads, d, block, ctx_len, hi,
                                           keep, n_policy_heads);
  if (out_bytes < total) return -1;
  std::memset(out, 0, static_cast<size_t>(total));
  std::vector<int64_t> hk, kk, b8, b4;
  kv_policy(n_q_heads, n_kv_heads, hi, keep, n_policy_heads, hk, kk);
  const int64_t c = (ctx_len - 1) / block;
  const int64_t dir = 64;
  int64_t data = (64 + 64 * static_cast<int64_t>(batch) * n_kv_heads + 255) / 256 * 256;
  put_i32(out + 0, 0x43564B54);  // "TKVC"
  put_i32(out + 4, 2);  // format version
  put_i32(out + 8, batch);
  put_i32(out + 12, n_kv_heads);
  put_i32(out + 16, d);
  put_i32(out + 20, block);
  put_i32(out + 24, static_cast<int32_t>(c + 1));
  put_i32(out + 28, static_cast<int32_t>(c));
  put_i64(out + 32, ctx_len);
  put_i64(out + 40, total);
  put_i64(out + 48, dir);
  put_i64(out + 56, data);
  int64_t off = data;
  for (int b = 0; b < batch; ++b)
    for (int g = 0; g < n_kv_heads; ++g) {
      stored_sets(c, hk[g], kk[g], b8, b4);
      int64_t lo8 = c;
      while (lo8 > 0 && std::find(b8.begin(), b8.end(), lo8 - 1) != b8.end()) --lo8;
      const int32_t sink = (lo8 > 0) ? 1 : 0;  // block 0 is always among b8
      uint8_t* e = out + dir + 64 * (static_cast<int64_t>(b) * n_kv_heads + g);
      put_i64(e + 0, off);
      put_i32(e + 8, static_cast<int32_t>(b8.size()));
      put_i32(e + 12, static_cast<int32_t>(b4.size()));
      put_i32(e + 16, static_cast<int32_t>(hk[g]));
      put_i32(e + 20, static_cast<int32_t>(kk[g]));
      put_i32(e + 24, static_cast<int32_t>(lo8));
      put_i32(e + 28, sink);
      put_i32(e + 32, b4.empty() ? 0 : static_cast<int32_t>(b4.front()));
      put_i32(e + 36, b4.empty() ? -1 : static_cast<int32_t>(b4.back()));
      const int64_t src = (static_cast<int64_t>(b) * n_kv_heads + g) * n;
      for (int pass = 0; pass < 2; ++pass) {
        const std::vector<int64_t>& blocks = pass == 0 ? b8 : b4;
        const int qmax = pass == 0 ? 127 : 7;
        const int64_t kbytes = pass == 0 ? static_cast<int64_t>(block) * d : static_cast<int64_t>(block) * d / 2;
        for (int64_t kb : blocks) {
          // codes and scales of the block's rows (rows at or past ctx_len stay zero)
          std::vector<int8_t> kcodes(static_cast<size_t>(block) * d, 0), vcodes(static_cast<size_t>(block) * d, 0);
          std::vector<float> kscale(block, 0.0f), vscale(block, 0.0f);
          for (int r = 0; r < block; ++r) {
            const int64_t tok = kb * block + r;
            if (tok >= ctx_len) continue;
            quantize_row(k + (src + tok) * d, d, qmax, &kcodes[static_cast<size_t>(r) * d], &kscale[r]);
            quantize_row(v + (src + tok) * d, d, qmax, &vcodes[static_cast<size_t>(r) * d], &vscale[r]);
          }
          write_record(kcodes.data(), vcodes.data(), kscale.data(), vscale.data(), block, d, pass == 1, out + off);
          off += 2 * kbytes + 8LL * block;
        }
      }
    }
  return 0;
}

// ============================================================ (5) decode
// One query token at t = ctx_len - 1 per sequence.  Works from the raw bf16 K/V
// and the policy (it never reads a packed cache): the stored set of block c, the
// query quantised at each precision, exact integer dots, softmax in double.
// The decode of every (b, h); masks (or null): per stored record, the query heads
// of its KV head that keep it (the dynamic skipping below).
static int decode_masked(int batch, int n_q_heads, int n_kv_heads, int d, int block, int64_t n, int64_t ctx_len,
                         const std::vector<int64_t>& hk, const std::vector<int64_t>& kk, const uint16_t* k,
                         const uint16_t* v, const uint16_t* q, float sm_scale, float* out, const uint32_t* masks,
                         int nthreads) {
  const int G = n_q_heads / n_kv_heads;
  const int64_t t_pos = ctx_len - 1, c = t_pos / block;
  parallel_for(static_cast<int64_t>(batch) * n_q_heads, nthreads, [&](int64_t bh) {
    const int b = static_cast<int>(bh / n_q_heads), h = static_cast<int>(bh % n_q_heads);
    const int g = h / G;
    std::vector<int8_t> qc8(d), qc4(d), kc(d), vc(d);
    float sq8, sq4, sk, sv;
    quantize_row(q + bh * d, d, 127, qc8.data(), &sq8);
    quantize_row(q + bh * d, d, 7, qc4.data(), &sq4);
    const int64_t src = (static_cast<int64_t>(b) * n_kv_heads + g) * n;
    // record index of each stored block (for the masks)
    std::vector<int64_t> rec_of(static_cast<size_t>(c + 1), -1), blocks;
    std::vector<int> qmaxs;
    record_order(c, hk[g], kk[g], blocks, qmaxs);
    for (size_t r = 0; r < blocks.size(); ++r) rec_of[static_cast<size_t>(blocks[r])] = static_cast<int64_t>(r);
    const int64_t pair_rec0 = (static_cast<int64_t>(b) * n_kv_heads + g) * (c + 1);
    std::vector<double> s;
    std::vector<int64_t> toks;
    std::vector<int> prec;
    for (int64_t j = 0; j <= t_pos; ++j) {
      const int a = tile_action(c, j / block, hk[g], kk[g]);
      if (a == ACT_SKIP) continue;
      if (masks && !((masks[pair_rec0 + rec_of[static_cast<size_t>(j / block)]] >> (h % G)) & 1u)) continue;
      const int qmax = a == ACT_INT8 ? 127 : 7;
      quantize_row(k + (src + j) * d, d, qmax, kc.data(), &sk);
      const int8_t* qc = a == ACT_INT8 ? qc8.data() : qc4.data();
      int64_t dot = 0;
      for (int x = 0; x < d; ++x) dot += static_cast<int64_t>(qc[x]) * kc[x];
      const double sqa = a == ACT_INT8 ? sq8 : sq4;
      s.push_back(static_cast<double>(dot) * sqa * sk * static_cast<double>(sm_scale));
      toks.push_back(j);
      prec.push_back(qmax);
    }
    const double mx = *std::max_element(s.begin(), s.end());
    std::vector<double> o(d, 0.0);
    double den = 0.0;
    for (size_t x = 0; x < s.size(); ++x) {
      const double p = std::exp(s[x] - mx);
      den += p;
      quantize_row(v + (src + toks[x]) * d, d, prec[x], vc.data(), &sv);
      for (int y = 0; y < d; ++y) o[y] += p * static_cast<double>(sv) * vc[y];
    }
    for (int y = 0; y < d; ++y) out[bh * d + y] = static_cast<float>(o[y] / den);
  });
  return 0;
}

int oracle_decode(int batch, int n_q_heads, int n_kv_heads, int d, int block, int64_t n,
                  int64_t ctx_len, const int32_t* hi, const int32_t* keep, int n_policy_heads,
                  const uint16_t* k, const uint16_t* v, const uint16_t* q, float sm_scale,
                  float* out, int nthreads) {
  std::vector<int64_t> hk, kk;
  kv_policy(n_q_heads, n_kv_heads, hi, keep, n_policy_heads, hk, kk);
  return decode_masked(batch, n_q_heads, n_kv_heads, d, block, n, ctx_len, hk, kk, k, v, q, sm_scale, out, nullptr,
                       nthreads);
}


// ---------------------------------------------------------------- calibration
// TriAttention summary page (rit.work), section on how calibration distributes
// compute between heads: a variant's cost counts whole processed blocks (the QK
// product, the weight normalisation and the value aggregation).  Here: every tile
// the rule keeps, counted one by one, as block*block pairs at its precision's cost.
double oracle_policy_cost(int64_t n, int block, int64_t hi, int64_t keep, double c8, double c4) {
  const int64_t nb = (n + block - 1) / block;
  int64_t t8 = 0, t4 = 0;
  for (int64_t qb = 0; qb < nb; ++qb)
    for (int64_t kb = 0; kb <= qb; ++kb) {
      const int a = tile_action(qb, kb, hi, keep);
      if (a == ACT_INT8) ++t8;
      if (a == ACT_INT4) ++t4;
    }
  return (c8 * (double)t8 + c4 * (double)t4) * ((double)block * (double)block);
}

// Same section: one global allocator grants more context or more precision where the
// added work lowers the error most.  Every head starts at (0, 0); at each step every
// head's two moves are looked at -- keep + 1 (one more block kept), hi + 1 (one more
// block at int8, keep raised with it when equal), both <= K -- and the move with the
// largest error reduction per added cost that fits the budget is applied (a reduction
// at no cost ranks above any ratio; ties: lower head, then the keep move); moves that
// reduce no error are not taken.  err[h][hi][keep], (K + 1) x (K + 1) per head.
// Returns 1 when the budget is below the protected-only cost, else 0.
int oracle_allocate_policy(int64_t n, int block, int H, int K, const double* err, double c8, double c4,
                           double budget, int32_t* hi, int32_t* keep, double* total_cost, double* total_err) {
  const int64_t S = K + 1;
  auto E = [&](int h, int64_t a, int64_t k) { return err[((int64_t)h * S + a) * S + k]; };
  auto cost = [&](int64_t a, int64_t k) { return oracle_policy_cost(n, block, a, k, c8, c4); };
  double total = 0.0;
  for (int h = 0; h < H; ++h) {
    hi[h] = 0;
    keep[h] = 0;
    total += cost(0, 0);
  }
  if (total > budget) return 1;
  for (;;) {
    bool found = false;
    int bh = 0, bm = 0;
    int64_t ba = 0, bk = 0;
    double bscore = 0.0, bdc = 0.0;
    for (int h = 0; h < H; ++h)
      for (int m = 0; m < 2; ++m) {
        int64_t a = hi[h], k = keep[h];
        if (m == 0) {
          if (k >= K) continue;
          k += 1;
        } else {
          if (a >= K) continue;
          a += 1;
          if (k < a) k = a;
        }
        const double de = E(h, hi[h], keep[h]) - E(h, a, k);
        if (!(de > 0.0)) continue;
        const double dc = cost(a, k) - cost(hi[h], keep[h]);
        if (total + dc > budget) continue;
        const double score = dc > 0.0 ? de / dc : INFINITY;
        // strictly better score wins; equal scores keep the earlier (head, move)
        if (!found || score > bscore) {
          found = true;
          bh = h;
          bm = m;
          ba = a;
          bk = k;
          bscore = score;
          bdc = dc;
        }
      }
    if (!found) break;
    (void)bm;
    total += bdc;
    hi[bh] = (int32_t)ba;
    keep[bh] = (int32_t)bk;
  }
  double es = 0.0;
  for (int h = 0; h < H; ++h) es += E(h, hi[h], keep[h]);
  *total_cost = total;
  *total_err = es;
  return 0;
}


// Statistics of every stored record (record order as in the cache; rmax = c + 1
// slots per pair, unused slots zero): lo, hi [P][rmax][d], smax, nmax [P][rmax].
int oracle_block_summaries(int batch, int n_q_heads, int n_kv_heads, int d, int block, int64_t n,
                           int64_t ctx_len, const int32_t* hi, const int32_t* keep, int n_policy_heads,
                           const uint16_t* k, int8_t* lo, int8_t* hi_out, float* smax, double* nmax,
                           int nthreads) {
  std::vector<int64_t> hk, kk;
  kv_policy(n_q_heads, n_kv_heads, hi, keep, n_policy_heads, hk, kk);
  const int64_t c = (ctx_len - 1) / block, rmax = c + 1;
  parallel_for(static_cast<int64_t>(batch) * n_kv_heads, nthreads, [&](int64_t p) {
    const int g = static_cast<int>(p % n_kv_heads);
    std::vector<int64_t> blocks;
    std::vector<int> qmaxs;
    record_order(c, hk[g], kk[g], blocks, qmaxs);
    const int64_t src = p * n;
    for (int64_t r = 0; r < rmax; ++r) {
      Summary s;
      if (r < static_cast<int64_t>(blocks.size()))
        s = summarise_block(k + (src + blocks[r] * block) * d, blocks[r] * block, ctx_len, block, d, qmaxs[r]);
      else {
        s.lo.assign(d, 0);
        s.hi.assign(d, 0);
      }
      std::memcpy(lo + (p * rmax + r) * d, s.lo.data(), static_cast<size_t>(d));
      std::memcpy(hi_out + (p * rmax + r) * d, s.hi.data(), static_cast<size_t>(d));
      smax[p * rmax + r] = s.smax;
      nmax[p * rmax + r] = s.nmax;
    }
  });
  return 0;
}

int oracle_skip_masks(int batch, int n_q_heads, int n_kv_heads, int d, int block, int64_t n, int64_t ctx_len,
                      const int32_t* hi, const int32_t* keep, int n_policy_heads, const uint16_t* k,
                      const uint16_t* q, const float* thresholds, float sm_scale, uint32_t* masks, int nthreads) {
  if (n_q_heads / n_kv_heads > 32) return -1;
  std::vector<int64_t> hk, kk;
  kv_policy(n_q_heads, n_kv_heads, hi, keep, n_policy_heads, hk, kk);
  skip_masks(batch, n_q_heads, n_kv_heads, d, block, n, ctx_len, hk, kk, k, q, thresholds, sm_scale, masks, nthreads);
  return 0;
}

// Decode with dynamic skipping: as oracle_decode, each query head attending only
// over the tokens of the stored blocks it keeps (the masks above).
int oracle_decode_skip(int batch, int n_q_heads, int n_kv_heads, int d, int block, int64_t n,
                       int64_t ctx_len, const int32_t* hi, const int32_t* keep, int n_policy_heads,
                       const uint16_t* k, const uint16_t* v, const uint16_t* q, const float* thresholds,
                       float sm_scale, float* out, int nthreads) {
  const int G = n_q_heads / n_kv_heads;
  if (G > 32) return -1;
  std::vector<int64_t> hk, kk;
  kv_policy(n_q_heads, n_kv_heads, hi, keep, n_policy_heads, hk, kk);
  const int64_t c = (ctx_len - 1) / block, rmax = c + 1;
  std::vector<uint32_t> masks(static_cast<size_t>(batch) * n_kv_heads * rmax);
  skip_masks(batch, n_q_heads, n_kv_heads, d, block, n, ctx_len, hk, kk, k, q, thresholds, sm_scale, masks.data(),
             nthreads);
  return decode_masked(batch, n_q_heads, n_kv_heads, d, block, n, ctx_len, hk, kk, k, v, q, sm_scale, out,
                       masks.data(), nthreads);
}


// Page table of a paged cache for ctx_len (format of the library's contract, written
// out here from its definition): header {"TKVP", 4, batch, kv heads, d, block, c + 1,
// c; ctx_len, page bytes, n_pages, 0}, one 64-byte entry per pair {0, 0, n8, n4, hi,
// keep, lo8, sink, lo4, hi4, 0...}, then per pair c + 1 page ids in record order (-1
// past its records); a variable-length table also keeps each pair's ctx_len (entry
// words 10-11) and its slot's sequence id (words 12-13).  A record whose (block,
// precision) the old table stores keeps its page, unless its slot now holds a new
// sequence (shorter, or another id); every other takes the next free page; old
// records not kept release theirs, in pair and record order.  Returns pages taken,
// or -1 (too few free pages), -2 (released list too small).
int64_t oracle_paged_table(int batch, int n_q_heads, int n_kv_heads, int d, int block, int64_t ctx_len,
                           const int64_t* ctx_lens, const int64_t* seq_ids, const int32_t* hi, const int32_t* keep,
                           int n_policy_heads,
                           int64_t n_pages, const uint8_t* old_table, const int32_t* free_pages, int64_t n_free,
                           uint8_t* table, int32_t* released, int64_t released_cap, int64_t* n_released) {
  std::vector<int64_t> hk, kk;
  kv_policy(n_q_heads, n_kv_heads, hi, keep, n_policy_heads, hk, kk);
  const int64_t P = static_cast<int64_t>(batch) * n_kv_heads;
  // each sequence's length (variable-length tables: ctx_lens[b]) and the widest one
  auto ctx_of = [&](int64_t p) { return ctx_lens ? ctx_lens[p / n_kv_heads] : ctx_len; };
  int64_t rmax = 0;
  for (int64_t p = 0; p < P; ++p) rmax = std::max(rmax, (ctx_of(p) - 1) / block + 1);
  int64_t orm = 0;
  if (old_table) {
    int32_t v;
    std::memcpy(&v, old_table + 24, 4);
    orm = v;
  }
  const int64_t bytes = 64 + 64 * P + 4 * P * rmax;
  std::memset(table, 0, static_cast<size_t>(bytes));
  int64_t taken = 0, nrel = 0;
  for (int64_t p = 0; p < P; ++p) {
    const int g = static_cast<int>(p % n_kv_heads);
    const int64_t ctx = ctx_of(p), c = (ctx - 1) / block;
    std::vector<int64_t> blocks, oblocks;
    std::vector<int> qm, oqm;
    record_order(c, hk[g], kk[g], blocks, qm);
    // the slot's sequence id (variable-length tables; 0 when none is given)
    const int64_t sid = ctx_lens && seq_ids ? seq_ids[p / n_kv_heads] : 0;
    int64_t octx = 0, osid = 0;
    if (old_table) {
      if (ctx_lens) {
        std::memcpy(&octx, old_table + 64 + 64 * p + 40, 8);
        std::memcpy(&osid, old_table + 64 + 64 * p + 48, 8);
      } else {
        std::memcpy(&octx, old_table + 32, 8);
      }
      record_order((octx - 1) / block, hk[g], kk[g], oblocks, oqm);
    }
    // a shorter sequence, or one with another id, is a new sequence in the slot
    const bool fresh = old_table && (ctx < octx || sid != osid);
    std::vector<int32_t> opages(oblocks.size());
    for (size_t o = 0; o < oblocks.size(); ++o)
      std::memcpy(&opages[o], old_table + 64 + 64 * P + 4 * (p * orm + static_cast<int64_t>(o)), 4);
    std::vector<bool> kept(oblocks.size(), false);
    for (int64_t r = 0; r < rmax; ++r) {
      int32_t pg = -1;
      if (r < static_cast<int64_t>(blocks.size())) {
        for (size_t o = 0; o < oblocks.size() && !fresh; ++o)
          if (oblocks[o] == blocks[r] && oqm[o] == qm[r] && !kept[o]) {
            pg = opages[o];
            kept[o] = true;
            break;
          }
        if (pg < 0) {
          if (taken >= n_free) return -1;
          pg = free_pages[taken++];
        }
      }
      put_i32(table + 64 + 64 * P + 4 * (p * rmax + r), pg);
    }
    for (size_t o = 0; o < oblocks.size(); ++o)
      if (!kept[o]) {
        if (nrel >= released_cap) return -2;
        released[nrel++] = opages[o];
      }
    std::vector<int64_t> b8, b4;
    stored_sets(c, hk[g], kk[g], b8, b4);
    int64_t lo8 = c;
    while (lo8 > 0 && std::find(b8.begin(), b8.end(), lo8 - 1) != b8.end()) --lo8;
    uint8_t* e = table + 64 + 64 * p;
    put_i32(e + 8, static_cast<int32_t>(b8.size()));
    put_i32(e + 12, static_cast<int32_t>(b4.size()));
    put_i32(e + 16, static_cast<int32_t>(hk[g]));
    put_i32(e + 20, static_cast<int32_t>(kk[g]));
    put_i32(e + 24, static_cast<int32_t>(lo8));
    put_i32(e + 28, lo8 > 0 ? 1 : 0);
    put_i32(e + 32, b4.empty() ? 0 : static_cast<int32_t>(b4.front()));
    put_i32(e + 36, b4.empty() ? -1 : static_cast<int32_t>(b4.back()));
    if (ctx_lens) {
      put_i64(e + 40, ctx);
      put_i64(e + 48, sid);
    }
  }
  put_i32(table + 0, 0x50564B54);  // "TKVP"
  put_i32(table + 4, 4);
  put_i32(table + 8, batch);
  put_i32(table + 12, n_kv_heads);
  put_i32(table + 16, d);
  put_i32(table + 20, block);
  put_i32(table + 24, static_cast<int32_t>(rmax));
  put_i32(table + 28, ctx_lens ? -1 : static_cast<int32_t>(rmax - 1));
  put_i64(table + 32, ctx_lens ? 0 : ctx_len);
  put_i64(table + 40, 2LL * block * d + 8LL * block);
  put_i64(table + 48, n_pages);
  *n_released = nrel;
  return taken;
}

// The page pool a paged cache implies: every stored record (the bytes the contiguous
// cache writer produces for it) at its page.  pool: n_pages * page bytes, pages not in
// the table left as they are.
int oracle_pack_paged(int batch, int n_q_heads, int n_kv_heads, int d, int block, int64_t n, int64_t ctx_len,
                      const int64_t* ctx_lens, const int32_t* hi, const int32_t* keep, int n_policy_heads,
                      const uint16_t* k, const uint16_t* v, const uint8_t* table, uint8_t* pool, int64_t pool_bytes) {
  const int64_t P = static_cast<int64_t>(batch) * n_kv_heads, page = 2LL * block * d + 8LL * block;
  int32_t rmax;
  std::memcpy(&rmax, table + 24, 4);
  // one batch element at a time (its own length when the table is variable-length)
  for (int b = 0; b < batch; ++b) {
    const int64_t ctx = ctx_lens ? ctx_lens[b] : ctx_len;
    const int64_t total = oracle_cache_bytes(1, n_q_heads, n_kv_heads, d, block, ctx, hi, keep, n_policy_heads);
    std::vector<uint8_t> cache(static_cast<size_t>(total));
    const int64_t src = static_cast<int64_t>(b) * n_kv_heads * n * d;
    if (oracle_pack_cache(1, n_q_heads, n_kv_heads, d, block, n, ctx, hi, keep, n_policy_heads, k + src, v + src,
                          cache.data(), total))
      return -1;
    for (int g = 0; g < n_kv_heads; ++g) {
      const int64_t p = static_cast<int64_t>(b) * n_kv_heads + g;
      int64_t off;
      int32_t n8, n4;
      std::memcpy(&off, cache.data() + 64 + 64 * g, 8);
      std::memcpy(&n8, cache.data() + 64 + 64 * g + 8, 4);
      std::memcpy(&n4, cache.data() + 64 + 64 * g + 12, 4);
      for (int64_t r = 0; r < n8 + n4; ++r) {
        int32_t pg;
        std::memcpy(&pg, table + 64 + 64 * P + 4 * (p * rmax + r), 4);
        const int64_t rb = r < n8 ? 2LL * block * d + 8LL * block : static_cast<int64_t>(block) * d + 8LL * block;
        if (pg < 0 || (pg + 1) * page > pool_bytes) return -2;
        std::memcpy(pool + pg * page, cache.data() + off, static_cast<size_t>(rb));
        off += rb;
      }
    }
  }
  return 0;
}

}  // extern "C"
