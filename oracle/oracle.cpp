// CPU oracle for the paged KV-cache decode operator.
//
// TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
// call this file: only the test suite, the smoke check and the benchmark's
// CPU-baseline leg use it.  It shares no code, header, table or constant with
// the HIP library; it is plain, slow, fp64 C++17 written to be checked by eye
// against the pages it cites:
//
//   [P1] "PagedAttention: Mathematical Foundations, Virtual Memory Block
//        Allocation, and Zero-Waste KV Cache Serving" (llms.blog)
//   [P2] "Pytorch implementation of paper: Efficient Memory Management for
//        Large Language Model Serving with PagedAttention (2023)" (aishastr.live)
//   [P3] the 10100.com article on why vLLM retired PagedAttention
//
// Every routine below is pinned by a CPU test against something other than
// itself (closed forms, library conversions, brute force, worked examples).
//
// Readings where the pages are silent or disagree (each is also listed in the
// design notes of the repository):
//   * cache layout: K and V are both [num_blocks][num_kv_heads][block_size][head_dim],
//     i.e. [P1] sec. 3 / sec. 7 per-block [block_size, head_dim] tiles with a head axis;
//   * tokens at or beyond context_len never enter the arithmetic ([P1] eq. for A_ij
//     counts only min(B, i-(t-1)B) rows of a block; [P2] sec. 2 slices to context_len);
//   * only table entries j < ceil(n/B) are read ([P2] sec. 2 loop bound);
//   * context_len == 0 gives an all-zero output row (not covered by the pages);
//   * GQA: query head h reads KV head h / (Hq/Hkv) (the pages only name num_kv_heads);
//   * fp8 is OCP E4M3FN with a per-tensor scale ([P3] sec. 4 dequant-on-load).

#include <cmath>
#include <cstdint>
#include <cstring>
#include <cstddef>
#include <algorithm>
#include <limits>
#include <thread>
#include <vector>

namespace {

// dtype codes used at this file's C interface (independent of the library's enum)
enum : int { OR_F16 = 0, OR_BF16 = 1, OR_E4M3 = 2 };

// ---------------------------------------------------------------------------
// Number formats, decoded and encoded from their definitions.
// ---------------------------------------------------------------------------

// IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
double f16_decode(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0) v = std::ldexp((double)m, -24);                       // subnormal: m * 2^-24
  else if (e == 31) v = (m == 0) ? std::numeric_limits<double>::infinity()
                                 : std::numeric_limits<double>::quiet_NaN();
  else v = std::ldexp((double)(1024 + m), e - 25);                  // (1 + m/1024) * 2^(e-15)
  return s ? -v : v;
}

// bfloat16: the upper 16 bits of an IEEE binary32.
double bf16_decode(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// OCP 8-bit floating point, E4M3 ("E4M3FN"): 1 sign, 4 exponent (bias 7),
// 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN;
// there are no infinities; the largest finite magnitude is 1.75 * 2^8 = 448.
double e4m3_decode(uint8_t b) {
  int s = (b >> 7) & 1, e = (b >> 3) & 0xF, m = b & 7;
  double v;
  if (e == 15 && m == 7) return std::numeric_limits<double>::quiet_NaN();
  if (e == 0) v = std::ldexp((double)m / 8.0, -6);
  else v = std::ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

// Round a finite double to the nearest value (ties to even) of a binary format
// with p significand bits (including the hidden one) and minimum normal
// exponent emin.  No overflow handling here; callers decide.
double round_to_format(double x, int p, int emin) {
  if (x == 0.0) return x;
  int e;
  std::frexp(x, &e);          // |x| in [2^(e-1), 2^e)
  int exp = e - 1;             // unbiased exponent of x
  if (exp < emin) exp = emin;  // subnormal range: fixed quantum
  double quantum = std::ldexp(1.0, exp - (p - 1));
  double scaled = x / quantum;            // exact (power-of-two scaling)
  double r = std::nearbyint(scaled);      // default rounding mode: nearest, ties to even
  return r * quantum;
}

// Encode an exactly representable non-negative magnitude into (exponent field, mantissa field).
void encode_fields(double a, int p, int emin, int bias, int* ef, int* mf) {
  if (a == 0.0) { *ef = 0; *mf = 0; return; }
  int e;
  std::frexp(a, &e);
  int exp = e - 1;
  if (exp < emin) {  // subnormal
    *ef = 0;
    *mf = (int)(a / std::ldexp(1.0, emin - (p - 1)));
  } else {
    *ef = exp + bias;
    *mf = (int)(a / std::ldexp(1.0, exp - (p - 1))) - (1 << (p - 1));
  }
}

uint16_t f16_encode(double x) {  // RNE, overflow to infinity
  if (std::isnan(x)) return 0x7E00;
  uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  double a = std::fabs(x);
  if (std::isinf(a)) return sign | 0x7C00;
  double r = round_to_format(a, 11, -14);
  if (r > 65504.0) return sign | 0x7C00;
  int ef, mf;
  encode_fields(r, 11, -14, 15, &ef, &mf);
  return sign | (uint16_t)(ef << 10) | (uint16_t)mf;
}

uint16_t bf16_encode(double x) {  // RNE, overflow to infinity
  if (std::isnan(x)) return 0x7FC0;
  uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  double a = std::fabs(x);
  if (std::isinf(a)) return sign | 0x7F80;
  double r = round_to_format(a, 8, -126);
  const double bf16_max = std::ldexp(255.0, 120);  // (2 - 2^-7) * 2^127
  if (r > bf16_max) return sign | 0x7F80;
  int ef, mf;
  encode_fields(r, 8, -126, 127, &ef, &mf);
  return sign | (uint16_t)(ef << 7) | (uint16_t)mf;
}

// fp32 -> E4M3FN, round to nearest even, saturating to +-448; NaN stays NaN.
uint8_t e4m3_encode(float xf) {
  double x = (double)xf;
  if (std::isnan(x)) return std::signbit(x) ? 0xFF : 0x7F;
  uint8_t sign = std::signbit(x) ? 0x80 : 0;
  double a = std::fabs(x);
  if (std::isinf(a)) return sign | 0x7E;
  double r = round_to_format(a, 4, -6);
  if (r > 448.0) r = 448.0;
  int ef, mf;
  encode_fields(r, 4, -6, 7, &ef, &mf);
  return sign | (uint8_t)(ef << 3) | (uint8_t)mf;
}

double load_elem(const void* base, size_t idx, int dtype) {
  switch (dtype) {
    case OR_F16: return f16_decode(((const uint16_t*)base)[idx]);
    case OR_BF16: return bf16_decode(((const uint16_t*)base)[idx]);
    case OR_E4M3: return e4m3_decode(((const uint8_t*)base)[idx]);
  }
  return std::numeric_limits<double>::quiet_NaN();
}

// Dequantized cache element: fp16/bf16 exactly; e4m3 as (float)code_value * (float)scale
// in binary32 round-to-nearest, then widened ([P3] sec. 4: the stored fp8 value is scaled
// by the per-tensor k_scale / v_scale on load).
double dequant(const void* cache, size_t idx, int dtype, float scale) {
  if (dtype != OR_E4M3) return load_elem(cache, idx, dtype);
  float v = (float)e4m3_decode(((const uint8_t*)cache)[idx]);
  volatile float prod = v * scale;  // one binary32 multiply, no contraction
  return (double)prod;
}

size_t elem_size(int dtype) { return dtype == OR_E4M3 ? 1 : 2; }

int ceil_div(int a, int b) { return (a + b - 1) / b; }

struct DecodeArgs {
  const void* q; int q_dtype;
  const void* k; const void* v; int kv_dtype;
  float k_scale, v_scale;
  const int32_t* tables; const int32_t* ctx;
  int S, Hq, Hkv, d, B, MB;
  double scale;
};

// Offset of element i of token t's row for KV head g, through the block table.
size_t cache_index(const DecodeArgs& a, int s, int t, int g, int i) {
  int blk = a.tables[(size_t)s * a.MB + t / a.B];
  int off = t % a.B;
  return (((size_t)blk * a.Hkv + g) * a.B + off) * a.d + i;
}

// [P1] sec. 3, eq. for a_ij and o_i: o = sum_t softmax_t(scale * q.k_t) v_t over the
// context_len tokens of sequence s, each token's k/v reached through the block table.
void decode_row(const DecodeArgs& a, int s, int h, double* out, double* weights) {
  const int n = a.ctx[s];
  const int g = h / (a.Hq / a.Hkv);
  double* o = out + ((size_t)s * a.Hq + h) * a.d;
  for (int i = 0; i < a.d; ++i) o[i] = 0.0;
  if (n <= 0) return;
  const size_t qoff = ((size_t)s * a.Hq + h) * a.d;
  std::vector<double> z(n);
  for (int t = 0; t < n; ++t) {
    double dot = 0.0;
    for (int i = 0; i < a.d; ++i)
      dot += load_elem(a.q, qoff + i, a.q_dtype) *
             dequant(a.k, cache_index(a, s, t, g, i), a.kv_dtype, a.k_scale);
    z[t] = a.scale * dot;
  }
  double m = -std::numeric_limits<double>::infinity();
  for (int t = 0; t < n; ++t) m = std::max(m, z[t]);
  double Z = 0.0;
  for (int t = 0; t < n; ++t) { z[t] = std::exp(z[t] - m); Z += z[t]; }
  for (int t = 0; t < n; ++t) {
    double at = z[t] / Z;
    if (weights) weights[((size_t)s * a.Hq + h) * a.MB * a.B + t] = at;
    for (int i = 0; i < a.d; ++i)
      o[i] += at * dequant(a.v, cache_index(a, s, t, g, i), a.kv_dtype, a.v_scale);
  }
}

// [P1] sec. 7 decoding pseudocode, written from its description: walk the block
// table one block at a time, score the block, and fold it into a running maximum,
// a running denominator and a running output, rescaling both by exp(old max -
// new max).  Blocks are visited in the order given by `order` (a permutation of
// 0..nblk-1) and, following the partial-block rule of [P1] sec. 3, slots at or
// beyond context_len are left out of the block's scores.
void decode_row_online(const DecodeArgs& a, int s, int h, const int32_t* order, double* out) {
  const int n = a.ctx[s];
  const int g = h / (a.Hq / a.Hkv);
  double* o = out + ((size_t)s * a.Hq + h) * a.d;
  std::vector<double> acc(a.d, 0.0);
  for (int i = 0; i < a.d; ++i) o[i] = 0.0;
  if (n <= 0) return;
  const size_t qoff = ((size_t)s * a.Hq + h) * a.d;
  const int nblk = ceil_div(n, a.B);
  double running_max = -std::numeric_limits<double>::infinity();
  double running_sum = 0.0;
  std::vector<double> scores(a.B);
  for (int step = 0; step < nblk; ++step) {
    const int j = order ? order[step] : step;
    const int valid = std::min(a.B, n - j * a.B);
    double block_max = -std::numeric_limits<double>::infinity();
    for (int r = 0; r < valid; ++r) {
      double dot = 0.0;
      for (int i = 0; i < a.d; ++i)
        dot += load_elem(a.q, qoff + i, a.q_dtype) *
               dequant(a.k, cache_index(a, s, j * a.B + r, g, i), a.kv_dtype, a.k_scale);
      scores[r] = a.scale * dot;
      block_max = std::max(block_max, scores[r]);
    }
    const double new_max = std::max(running_max, block_max);
    const double rescale = std::exp(running_max - new_max);  // exp(-inf) = 0 on the first block
    double block_sum = 0.0;
    for (int i = 0; i < a.d; ++i) acc[i] *= rescale;
    for (int r = 0; r < valid; ++r) {
      const double p = std::exp(scores[r] - new_max);
      block_sum += p;
      for (int i = 0; i < a.d; ++i)
        acc[i] += p * dequant(a.v, cache_index(a, s, j * a.B + r, g, i), a.kv_dtype, a.v_scale);
    }
    running_sum = running_sum * rescale + block_sum;
    running_max = new_max;
  }
  for (int i = 0; i < a.d; ++i) o[i] = acc[i] / running_sum;
}

// Split the context into partitions of P tokens (P a multiple of B, partition p
// covering tokens [p*P, min(n, (p+1)*P))), run the online recurrence above inside
// each partition, then combine the partial states (m_p, l_p, acc_p) with the same
// rescaling rule: M = max_p m_p, L = sum_p l_p e^(m_p - M), o = sum_p acc_p e^(m_p - M) / L.
// The pages have no partition merge; this is the rescale step of [P1] sec. 7 applied
// once more across partitions.
void decode_row_partitioned(const DecodeArgs& a, int s, int h, int P, double* out) {
  const int n = a.ctx[s];
  const int g = h / (a.Hq / a.Hkv);
  double* o = out + ((size_t)s * a.Hq + h) * a.d;
  for (int i = 0; i < a.d; ++i) o[i] = 0.0;
  if (n <= 0) return;
  const size_t qoff = ((size_t)s * a.Hq + h) * a.d;
  const int nparts = ceil_div(n, P);
  std::vector<double> m(nparts), l(nparts), acc((size_t)nparts * a.d, 0.0);
  for (int p = 0; p < nparts; ++p) {
    const int t0 = p * P, t1 = std::min(n, t0 + P);
    double mx = -std::numeric_limits<double>::infinity();
    std::vector<double> z(t1 - t0);
    for (int t = t0; t < t1; ++t) {
      double dot = 0.0;
      for (int i = 0; i < a.d; ++i)
        dot += load_elem(a.q, qoff + i, a.q_dtype) *
               dequant(a.k, cache_index(a, s, t, g, i), a.kv_dtype, a.k_scale);
      z[t - t0] = a.scale * dot;
      mx = std::max(mx, z[t - t0]);
    }
    double sum = 0.0;
    for (int t = t0; t < t1; ++t) {
      const double w = std::exp(z[t - t0] - mx);
      sum += w;
      for (int i = 0; i < a.d; ++i)
        acc[(size_t)p * a.d + i] += w * dequant(a.v, cache_index(a, s, t, g, i), a.kv_dtype, a.v_scale);
    }
    m[p] = mx;
    l[p] = sum;
  }
  double M = -std::numeric_limits<double>::infinity();
  for (int p = 0; p < nparts; ++p) M = std::max(M, m[p]);
  double L = 0.0;
  for (int p = 0; p < nparts; ++p) L += l[p] * std::exp(m[p] - M);
  for (int i = 0; i < a.d; ++i) {
    double v = 0.0;
    for (int p = 0; p < nparts; ++p) v += acc[(size_t)p * a.d + i] * std::exp(m[p] - M);
    o[i] = v / L;
  }
}

// Several query tokens per sequence (speculative / tree verification, [P1] sec. 9 names
// speculative decoding trees among the uses of the shared block store).  Reading: the T
// query tokens of sequence s are its last T positions n-T .. n-1, already stored in the
// cache; query t sees every position before n-T and the draft position n-T+u iff bit u
// of its mask is set (causal mask: bits 0..t).  The output is the same softmax-weighted
// sum of [P1] sec. 3 over the visible positions; no visible position gives a zero row.
void decode_row_multi(const DecodeArgs& a, int T, const uint32_t* masks, int s, int t, int h,
                      double* out) {
  const int n = a.ctx[s];
  const int g = h / (a.Hq / a.Hkv);
  const size_t row = ((size_t)s * T + t) * a.Hq + h;
  double* o = out + row * a.d;
  for (int i = 0; i < a.d; ++i) o[i] = 0.0;
  const uint32_t mask = masks ? masks[(size_t)s * T + t] : (uint32_t)((2ull << t) - 1);
  const int first_draft = n - T;
  std::vector<int> vis;
  for (int p = 0; p < n; ++p) {
    if (p < first_draft) { vis.push_back(p); continue; }
    const int u = p - first_draft;
    if (u < 32 && ((mask >> u) & 1u)) vis.push_back(p);
  }
  if (vis.empty()) return;
  std::vector<double> z(vis.size());
  for (size_t k = 0; k < vis.size(); ++k) {
    double dot = 0.0;
    for (int i = 0; i < a.d; ++i)
      dot += load_elem(a.q, row * a.d + i, a.q_dtype) *
             dequant(a.k, cache_index(a, s, vis[k], g, i), a.kv_dtype, a.k_scale);
    z[k] = a.scale * dot;
  }
  double m = -std::numeric_limits<double>::infinity();
  for (double x : z) m = std::max(m, x);
  double Z = 0.0;
  for (double& x : z) { x = std::exp(x - m); Z += x; }
  for (size_t k = 0; k < vis.size(); ++k)
    for (int i = 0; i < a.d; ++i)
      o[i] += z[k] / Z * dequant(a.v, cache_index(a, s, vis[k], g, i), a.kv_dtype, a.v_scale);
}

template <class F>
void parallel_rows(int nrows, int threads, F&& f) {
  if (threads <= 1 || nrows <= 1) {
    for (int r = 0; r < nrows; ++r) f(r);
    return;
  }
  threads = std::min(threads, nrows);
  std::vector<std::thread> pool;
  for (int w = 0; w < threads; ++w)
    pool.emplace_back([&, w] { for (int r = w; r < nrows; r += threads) f(r); });
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

// ---- scalar conversions (exported for the pins) ----
double or_f16_to_f64(uint16_t h) { return f16_decode(h); }
double or_bf16_to_f64(uint16_t b) { return bf16_decode(b); }
double or_e4m3_to_f64(uint8_t b) { return e4m3_decode(b); }
uint16_t or_f64_to_f16(double x) { return f16_encode(x); }
uint16_t or_f64_to_bf16(double x) { return bf16_encode(x); }
uint8_t or_f32_to_e4m3(float x) { return e4m3_encode(x); }

void or_f64_to_dtype_array(const double* x, size_t n, int dtype, void* out) {
  for (size_t i = 0; i < n; ++i) {
    if (dtype == OR_F16) ((uint16_t*)out)[i] = f16_encode(x[i]);
    else if (dtype == OR_BF16) ((uint16_t*)out)[i] = bf16_encode(x[i]);
    else ((uint8_t*)out)[i] = e4m3_encode((float)x[i]);
  }
}

void or_dequant_array(const void* src, size_t n, int dtype, float scale, double* out) {
  for (size_t i = 0; i < n; ++i) out[i] = dequant(src, i, dtype, scale);
}

// ---- O1: block tables from a free list ----
// [P1] sec. 4 allocation lifecycle and [P2] sec. 3 BlockManager: a prompt of N tokens
// takes ceil(N/B) blocks popped from the front of the free list; a finished
// sequence's blocks are returned to the back.  [P1] sec. 5 parallel sampling: a
// prompt shared by K sequences is stored once in blocks whose reference count is K.
//
// Sequences are processed in index order.  Sequence s in prefix group g (prefix_group[s]
// = g >= 0) first takes the group's floor(prefix_lens[g] / B) shared blocks (popped when
// the group is first met), then pops its remaining ceil(n_s/B) - shared private blocks.
// Table rows are padded with -1.  refcounts[id] = number of rows that reference id.
// On success free_list/free_count are updated in place and 0 is returned.  If the pool
// is too small, or a row would exceed max_blocks, or a grouped sequence is shorter than
// its prefix, nothing is changed and a negative value is returned (-3: no blocks,
// -4: table overflow, -1: invalid argument).
int or_build_tables(int32_t* free_list, int32_t* free_count, int32_t block_size,
                    int32_t num_seqs, const int32_t* context_lens,
                    const int32_t* prefix_group, const int32_t* prefix_lens, int32_t num_groups,
                    int32_t max_blocks, int32_t* tables, int32_t* refcounts, int32_t num_blocks) {
  if (block_size < 1 || num_seqs < 0 || max_blocks < 1) return -1;
  // First a dry run: count the blocks needed, check every row fits.
  std::vector<char> group_seen(std::max(num_groups, 0), 0);
  long needed = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int n = context_lens[s];
    if (n < 0) return -1;
    const int total = ceil_div(n, block_size);
    if (total > max_blocks) return -4;
    int shared = 0;
    if (prefix_group && prefix_group[s] >= 0) {
      const int g = prefix_group[s];
      if (g >= num_groups) return -1;
      if (prefix_lens[g] > n) return -1;
      shared = prefix_lens[g] / block_size;
      if (!group_seen[g]) { needed += shared; group_seen[g] = 1; }
    }
    needed += total - shared;
  }
  if (needed > *free_count) return -3;

  // Real run.
  std::vector<int32_t> fl(free_list, free_list + *free_count);
  size_t head = 0;
  std::vector<std::vector<int32_t>> group_blocks(std::max(num_groups, 0));
  std::fill(group_seen.begin(), group_seen.end(), 0);
  for (int s = 0; s < num_seqs; ++s) {
    int32_t* row = tables + (size_t)s * max_blocks;
    for (int j = 0; j < max_blocks; ++j) row[j] = -1;
    const int total = ceil_div(context_lens[s], block_size);
    int j = 0;
    if (prefix_group && prefix_group[s] >= 0) {
      const int g = prefix_group[s];
      const int shared = prefix_lens[g] / block_size;
      if (!group_seen[g]) {
        for (int k = 0; k < shared; ++k) group_blocks[g].push_back(fl[head++]);
        group_seen[g] = 1;
      }
      for (; j < shared; ++j) row[j] = group_blocks[g][j];
    }
    for (; j < total; ++j) row[j] = fl[head++];
  }
  // Remaining free list keeps its order.
  const int32_t remain = (int32_t)(fl.size() - head);
  for (int32_t k = 0; k < remain; ++k) free_list[k] = fl[head + k];
  *free_count = remain;
  if (refcounts) {
    for (int b = 0; b < num_blocks; ++b) refcounts[b] = 0;
    for (int s = 0; s < num_seqs; ++s)
      for (int j = 0; j < max_blocks; ++j) {
        const int32_t id = tables[(size_t)s * max_blocks + j];
        if (id >= 0) refcounts[id] += 1;
      }
  }
  return 0;
}

// Release the rows `seqs` of `tables`: each referenced block's count drops by one and
// a block reaching zero is appended to the back of the free list, in row order
// ([P1] sec. 4 completion; [P2] sec. 3 free extends the free list).
void or_free_rows(int32_t* free_list, int32_t* free_count, const int32_t* tables,
                  int32_t max_blocks, int32_t n, const int32_t* seqs, int32_t* refcounts) {
  for (int k = 0; k < n; ++k) {
    const int32_t* row = tables + (size_t)seqs[k] * max_blocks;
    for (int j = 0; j < max_blocks; ++j) {
      const int32_t id = row[j];
      if (id < 0) continue;
      refcounts[id] -= 1;
      if (refcounts[id] == 0) free_list[(*free_count)++] = id;
    }
  }
}

// ---- O2: scatter new tokens into their slots ----
// [P1] sec. 4 decoding step and sec. 7 fused block write: token t of sequence
// seq_ids[t] at position positions[t] lands in block tables[seq][pos / B], slot
// pos % B.  Same-dtype caches receive the source bits unchanged; an e4m3 cache
// receives e4m3(float(src) * inv_scale) (binary32 multiply, RNE, saturating).
void or_scatter(const void* src, int src_dtype, void* cache, int cache_dtype,
                const int32_t* tables, int32_t max_blocks,
                const int32_t* seq_ids, const int32_t* positions, int32_t num_tokens,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float inv_scale) {
  for (int t = 0; t < num_tokens; ++t) {
    const int32_t blk = tables[(size_t)seq_ids[t] * max_blocks + positions[t] / block_size];
    const int32_t off = positions[t] % block_size;
    for (int h = 0; h < num_kv_heads; ++h)
      for (int i = 0; i < head_dim; ++i) {
        const size_t si = ((size_t)t * num_kv_heads + h) * head_dim + i;
        const size_t di = (((size_t)blk * num_kv_heads + h) * block_size + off) * head_dim + i;
        if (cache_dtype == src_dtype) {
          ((uint16_t*)cache)[di] = ((const uint16_t*)src)[si];
        } else {  // e4m3 cache from an fp16/bf16 source
          const float x = (float)load_elem(src, si, src_dtype);
          volatile float scaled = x * inv_scale;
          ((uint8_t*)cache)[di] = e4m3_encode(scaled);
        }
      }
  }
}

// ---- O4: the decode output in fp64 ----
// rows == nullptr: every (s, h); otherwise nrows pairs rows[2r] = s, rows[2r+1] = h.
// out is [S, Hq, d] doubles (only the listed rows are written when rows is given).
// weights, if non-null, is [S, Hq, max_blocks * B] and receives a_t for t < n.
void or_decode(const void* q, int q_dtype, const void* k_cache, const void* v_cache, int kv_dtype,
               float k_scale, float v_scale, const int32_t* tables, const int32_t* context_lens,
               int32_t S, int32_t Hq, int32_t Hkv, int32_t d, int32_t B, int32_t MB, float scale,
               const int32_t* rows, int32_t nrows, int32_t threads, double* out, double* weights) {
  DecodeArgs a{q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, tables, context_lens,
               S, Hq, Hkv, d, B, MB, (double)scale};
  if (!rows) {
    parallel_rows(S * Hq, threads, [&](int r) { decode_row(a, r / Hq, r % Hq, out, weights); });
  } else {
    parallel_rows(nrows, threads, [&](int r) { decode_row(a, rows[2 * r], rows[2 * r + 1], out, weights); });
  }
}

// The pages' block-at-a-time online recurrence (pinned against or_decode).
// block_orders, if non-null, is [S, MB]: row s lists the visiting order of its blocks.
void or_decode_online(const void* q, int q_dtype, const void* k_cache, const void* v_cache, int kv_dtype,
                      float k_scale, float v_scale, const int32_t* tables, const int32_t* context_lens,
                      int32_t S, int32_t Hq, int32_t Hkv, int32_t d, int32_t B, int32_t MB, float scale,
                      const int32_t* block_orders, double* out) {
  DecodeArgs a{q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, tables, context_lens,
               S, Hq, Hkv, d, B, MB, (double)scale};
  for (int s = 0; s < S; ++s)
    for (int h = 0; h < Hq; ++h)
      decode_row_online(a, s, h, block_orders ? block_orders + (size_t)s * MB : nullptr, out);
}

// Partitioned recurrence with the cross-partition merge (pinned against or_decode).
void or_decode_partitioned(const void* q, int q_dtype, const void* k_cache, const void* v_cache,
                           int kv_dtype, float k_scale, float v_scale, const int32_t* tables,
                           const int32_t* context_lens, int32_t S, int32_t Hq, int32_t Hkv,
                           int32_t d, int32_t B, int32_t MB, float scale, int32_t P, double* out) {
  DecodeArgs a{q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, tables, context_lens,
               S, Hq, Hkv, d, B, MB, (double)scale};
  for (int s = 0; s < S; ++s)
    for (int h = 0; h < Hq; ++h) decode_row_partitioned(a, s, h, P, out);
}

// Multi-token queries: q and out are [S, T, Hq, d]; tree_masks is [S, T] or null (causal).
void or_decode_multi(const void* q, int q_dtype, const void* k_cache, const void* v_cache,
                     int kv_dtype, float k_scale, float v_scale, const int32_t* tables,
                     const int32_t* context_lens, int32_t S, int32_t Hq, int32_t Hkv, int32_t d,
                     int32_t B, int32_t MB, float scale, int32_t T, const uint32_t* tree_masks,
                     int32_t threads, double* out) {
  DecodeArgs a{q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, tables, context_lens,
               S, Hq, Hkv, d, B, MB, (double)scale};
  parallel_rows(S * T * Hq, threads, [&](int r) {
    decode_row_multi(a, T, tree_masks, r / (T * Hq), (r / Hq) % T, r % Hq, out);
  });
}

// ---- O6: footprint ----
// [P1] sec. 1: each token stores a key and a value vector per layer; with
// num_kv_heads * head_dim values per vector and e bytes per value this is
// 2 * L * Hkv * d * e bytes (for fp16 and Hkv * d = d_model: 4 * L * d_model).
uint64_t or_kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim,
                               int32_t kv_dtype) {
  return 2ull * (uint64_t)num_layers * (uint64_t)num_kv_heads * (uint64_t)head_dim *
         (uint64_t)elem_size(kv_dtype);
}

}  // extern "C"
