// The decode C ABI called from C++ alone: device memory from hipMalloc, no
// Python or torch. Inputs come from a small counter-based generator, and every
// expected value comes from a case whose result has a closed form:
//  - equal keys within each (sequence, KV head): every score is equal, so each
//    query head of the group gets the mean of the V rows ("From Attention to
//    KV Cache Compression: Notes from a KernelGen Optimization", "Starting
//    from Attention": softmax of equal scores is uniform);
//  - one token per sequence: the softmax weight is 1, so the output is that
//    token's V row, bit for bit in bf16 and in fp32.
// Page slots no token uses, and a spare page the block tables point past the
// sequence end, hold NaN: any read through a wrong address shows up. The rows
// go through a shuffled block table ("海光 DCU 上的长上下文 Attention：从 page784
// 到 page832 的 KV Cache 对齐与访存优化", §1: logical page t / B, offset t % B).
// Also checked: host-side status codes, and pkv_decode_noalloc giving the same
// bits as pkv_decode. Prints one line per case; exit status 0 when all pass.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <utility>
#include <vector>

#include "pkv.h"

namespace {

constexpr int kHkv = 4, kHq = 24, kD = 256;
constexpr uint16_t kNaN = 0x7FC0;

int failures = 0;

#define CHECK_HIP(x)                                                              \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      std::exit(2);                                                               \
    }                                                                             \
  } while (0)

void expect(bool ok, const char* what) {
  std::printf("%s: %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++failures;
}

// splitmix64: the generator's output for counter i
uint64_t mix(uint64_t i) {
  uint64_t z = i + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
// uniform in [-1, 1)
float unit(uint64_t i) { return static_cast<float>((mix(i) >> 40) * (2.0 / 16777216.0) - 1.0); }

uint16_t to_bf16(float f) {   // round to nearest even (finite inputs)
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
float from_bf16(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

struct Case {
  std::vector<int> lens;
  int bsz = 0;
  int pool = 0;                       // pages holding tokens and NaN, plus one NaN page
  int max_blocks = 0;
  std::vector<uint16_t> q, k, v;      // q [S, Hq, D]; k, v [pool, B, Hkv, D]
  std::vector<int32_t> table;         // [S, max_blocks]
  std::vector<double> ref;            // [S, Hq, D]
};

// Sequence s: token t of KV head g has K row key(s, g) (equal keys) and a
// random V row; lens[s] == 1 makes the output that one V row whatever K is.
Case make_case(const std::vector<int>& lens, int bsz, uint64_t seed) {
  Case c;
  c.lens = lens;
  c.bsz = bsz;
  const int S = static_cast<int>(lens.size());
  int used = 0;
  for (int n : lens) {
    c.max_blocks = std::max(c.max_blocks, (n + bsz - 1) / bsz);
    used += (n + bsz - 1) / bsz;
  }
  c.max_blocks = std::max(c.max_blocks, 1);
  c.pool = used + 2;
  const size_t page = static_cast<size_t>(bsz) * kHkv * kD;
  c.k.assign(page * c.pool, kNaN);
  c.v.assign(page * c.pool, kNaN);
  c.q.resize(static_cast<size_t>(S) * kHq * kD);
  for (size_t i = 0; i < c.q.size(); ++i) c.q[i] = to_bf16(unit(seed * 1000003 + i));
  // a shuffled order of the pool's first `used` + 1 pages; the last page stays NaN
  std::vector<int> perm(c.pool - 1);
  for (int i = 0; i < c.pool - 1; ++i) perm[i] = i;
  for (int i = c.pool - 2; i > 0; --i) std::swap(perm[i], perm[mix(seed + 17 * i) % (i + 1)]);
  const int pad_page = c.pool - 1;
  c.table.assign(static_cast<size_t>(S) * c.max_blocks, pad_page);
  c.ref.assign(static_cast<size_t>(S) * kHq * kD, 0.0);
  int next = 0;
  for (int s = 0; s < S; ++s) {
    const int n = lens[s];
    for (int lp = 0; lp < (n + bsz - 1) / bsz; ++lp) c.table[s * c.max_blocks + lp] = perm[next++];
    std::vector<double> sum(static_cast<size_t>(kHkv) * kD, 0.0);
    for (int t = 0; t < n; ++t) {
      const size_t row = static_cast<size_t>(c.table[s * c.max_blocks + t / bsz]) * page +
                         static_cast<size_t>(t % bsz) * kHkv * kD;
      for (int g = 0; g < kHkv; ++g)
        for (int d = 0; d < kD; ++d) {
          const size_t at = row + static_cast<size_t>(g) * kD + d;
          c.k[at] = to_bf16(unit((seed << 20) + (static_cast<uint64_t>(s) * kHkv + g) * kD + d));
          const uint16_t vb = to_bf16(unit((seed << 40) + at));
          c.v[at] = vb;
          sum[static_cast<size_t>(g) * kD + d] += from_bf16(vb);
        }
    }
    for (int h = 0; h < kHq; ++h)
      for (int d = 0; d < kD; ++d)
        c.ref[(static_cast<size_t>(s) * kHq + h) * kD + d] =
            n > 0 ? sum[static_cast<size_t>(h / 6) * kD + d] / n : 0.0;
  }
  return c;
}

pkv_decode_params params_of(const Case& c, int partition_tokens) {
  pkv_decode_params p;
  std::memset(&p, 0, sizeof(p));
  p.num_seqs = static_cast<int32_t>(c.lens.size());
  p.num_q_heads = kHq;
  p.num_kv_heads = kHkv;
  p.head_size = kD;
  p.block_size = c.bsz;
  p.max_blocks_per_seq = c.max_blocks;
  p.k_page_stride = static_cast<int64_t>(c.bsz) * kHkv * kD;
  p.v_page_stride = p.k_page_stride;
  int mx = 1;
  for (int n : c.lens) mx = std::max(mx, n);
  p.max_seq_len = mx;
  p.partition_tokens = partition_tokens;
  p.scale = 1.0f / 16.0f;
  return p;
}

template <typename T>
T* to_device(const std::vector<T>& h) {
  T* d = nullptr;
  CHECK_HIP(hipMalloc(&d, std::max<size_t>(h.size(), 1) * sizeof(T)));
  if (!h.empty()) CHECK_HIP(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
  return d;
}

struct Outputs {
  std::vector<uint16_t> bf16;
  std::vector<float> f32;
};

// One pkv_decode (or pkv_decode_noalloc) call; the status goes to *status.
Outputs run(const Case& c, int partition_tokens, bool noalloc, int* status) {
  const pkv_decode_params p = params_of(c, partition_tokens);
  const size_t n_out = c.q.size();
  uint16_t* q = to_device(c.q);
  uint16_t* k = to_device(c.k);
  uint16_t* v = to_device(c.v);
  int32_t* table = to_device(c.table);
  std::vector<int32_t> lens(c.lens.begin(), c.lens.end());
  int32_t* sl = to_device(lens);
  uint16_t* out = nullptr;
  float* out32 = nullptr;
  CHECK_HIP(hipMalloc(&out, n_out * 2));
  CHECK_HIP(hipMalloc(&out32, n_out * 4));
  const size_t ws_bytes = pkv_decode_workspace_bytes(&p);
  void* ws = nullptr;
  if (!noalloc && ws_bytes > 0) CHECK_HIP(hipMalloc(&ws, ws_bytes));
  *status = noalloc ? pkv_decode_noalloc(&p, q, k, v, table, sl, out, out32, nullptr)
                    : pkv_decode(&p, q, k, v, table, sl, out, out32, ws, ws_bytes, nullptr);
  CHECK_HIP(hipDeviceSynchronize());
  Outputs o;
  o.bf16.resize(n_out);
  o.f32.resize(n_out);
  CHECK_HIP(hipMemcpy(o.bf16.data(), out, n_out * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(o.f32.data(), out32, n_out * 4, hipMemcpyDeviceToHost));
  for (void* ptr : {static_cast<void*>(q), static_cast<void*>(k), static_cast<void*>(v),
                    static_cast<void*>(table), static_cast<void*>(sl), static_cast<void*>(out),
                    static_cast<void*>(out32), ws})
    if (ptr) CHECK_HIP(hipFree(ptr));
  return o;
}

// bf16: |out - ref| <= 1e-2 + 1e-2 |ref| for every element; fp32: per (sequence,
// head) row, max |out - ref| <= 1e-4 max |ref| (and exact zeros for empty rows)
bool close_to_ref(const Case& c, const Outputs& o) {
  for (size_t row = 0; row < c.ref.size() / kD; ++row) {
    double mref = 0.0, err = 0.0;
    for (int d = 0; d < kD; ++d) {
      const size_t i = row * kD + d;
      const double r = c.ref[i];
      const double b = from_bf16(o.bf16[i]);
      if (!std::isfinite(b) || std::fabs(b - r) > 1e-2 + 1e-2 * std::fabs(r)) return false;
      mref = std::max(mref, std::fabs(r));
      err = std::max(err, std::fabs(static_cast<double>(o.f32[i]) - r));
    }
    if (!(err <= 1e-4 * mref)) return false;
  }
  return true;
}

}  // namespace

int main() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    std::printf("no GPU\n");
    return 2;
  }
  CHECK_HIP(hipSetDevice(0));
  std::printf("%s\n", pkv_version());

  // equal keys: the balanced split (several sequences, P = 0), fixed
  // partitions (P = 256), and page784
  {
    const Case c = make_case({1000, 70, 833, 0, 2500}, 832, 11);
    int st = -100;
    const Outputs a = run(c, 0, false, &st);
    expect(st == PKV_OK && close_to_ref(c, a), "equal keys, balanced split, page 832");
    const Outputs b = run(c, 256, false, &st);
    expect(st == PKV_OK && close_to_ref(c, b), "equal keys, fixed partitions of 256, page 832");
    const Outputs n = run(c, 0, true, &st);
    expect(st == PKV_OK && n.bf16 == a.bf16 &&
               std::memcmp(n.f32.data(), a.f32.data(), a.f32.size() * 4) == 0,
           "pkv_decode_noalloc gives pkv_decode's bits");
    const Case c784 = make_case({1000, 70, 833, 0, 2500}, 784, 11);
    const Outputs d = run(c784, 0, false, &st);
    expect(st == PKV_OK && close_to_ref(c784, d), "equal keys, balanced split, page 784");
  }
  // one long sequence (automatic fixed partitions) and one token per sequence
  {
    const Case c = make_case({9000}, 832, 12);
    int st = -100;
    const Outputs o9 = run(c, 0, false, &st);
    expect(st == PKV_OK && close_to_ref(c, o9), "equal keys, one sequence of 9000 tokens");
    const Case one = make_case({1, 1, 1}, 64, 13);
    const Outputs o = run(one, 0, false, &st);
    bool exact = st == PKV_OK;
    for (size_t i = 0; i < one.ref.size() && exact; ++i)
      exact = o.bf16[i] == to_bf16(static_cast<float>(one.ref[i])) &&
              o.f32[i] == static_cast<float>(one.ref[i]);
    expect(exact, "one token per sequence returns its V row bit for bit");
  }
  // host-side checks: status codes before any launch
  {
    const Case c = make_case({100}, 832, 14);
    pkv_decode_params p = params_of(c, 0);
    expect(pkv_decode(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                      nullptr, 0, nullptr) == PKV_ERR_NULL,
           "null params: PKV_ERR_NULL");
    pkv_decode_params bad = p;
    bad.block_size = 100;
    pkv_plan_info info;
    expect(pkv_plan(&bad, &info) == PKV_ERR_BLOCK_SIZE, "block size 100: PKV_ERR_BLOCK_SIZE");
    bad = p;
    bad.head_size = 128;
    expect(pkv_plan(&bad, &info) == PKV_ERR_UNSUPPORTED, "head size 128: PKV_ERR_UNSUPPORTED");
    bad = p;
    bad.partition_tokens = 100;
    expect(pkv_plan(&bad, &info) == PKV_ERR_PARTITION, "partition of 100: PKV_ERR_PARTITION");
    // a workspace declared one byte short is refused before any launch (the
    // buffers are real and the workspace full size, so nothing could go out
    // of bounds even if it were not)
    bad = p;
    bad.partition_tokens = 64;   // 2 partitions: a workspace is needed
    const size_t need = pkv_decode_workspace_bytes(&bad);
    uint16_t* q = to_device(c.q);
    uint16_t* k = to_device(c.k);
    uint16_t* v = to_device(c.v);
    int32_t* table = to_device(c.table);
    int32_t* sl = to_device(std::vector<int32_t>(c.lens.begin(), c.lens.end()));
    uint16_t* out = to_device(std::vector<uint16_t>(c.q.size(), 0));
    void* ws = nullptr;
    CHECK_HIP(hipMalloc(&ws, std::max<size_t>(need, 256)));
    expect(need > 0 && pkv_decode(&bad, q, k, v, table, sl, out, nullptr, ws, need - 1,
                                  nullptr) == PKV_ERR_WORKSPACE,
           "short workspace: PKV_ERR_WORKSPACE");
    CHECK_HIP(hipDeviceSynchronize());
    for (void* ptr : {static_cast<void*>(q), static_cast<void*>(k), static_cast<void*>(v),
                      static_cast<void*>(table), static_cast<void*>(sl),
                      static_cast<void*>(out), ws})
      CHECK_HIP(hipFree(ptr));
    expect(std::strlen(pkv_status_string(PKV_ERR_WORKSPACE)) > 0, "status strings");
  }
  std::printf("%s\n", failures == 0 ? "all passed" : "FAILED");
  return failures == 0 ? 0 : 1;
}
