// Host sanitizer driver for the CPU oracle (test infrastructure, like the oracle itself).
//
// Compiled together with sparse_mqa_oracle.cpp under AddressSanitizer + UndefinedBehaviorSanitizer
// or ThreadSanitizer (tests/test_oracle_sanitizers.py), it calls every exported oracle function,
// in both precisions, on small inputs that reach each branch: out-of-range indices of every kind
// (negative, INT32_MIN, S_kv, INT32_MAX), a token selecting one row twice, a fully masked token, a
// -inf sink, explicit token and row lists, and a ragged topk. It checks that outputs are finite
// where the definition makes them finite and exits non-zero otherwise; the sanitizers report
// invalid accesses, undefined behaviour and data races on their own.
#include "sparse_mqa_oracle.cpp"

#include <cstdio>
#include <random>

namespace {

template <class R>
int run_case(int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk, uint32_t seed) {
  std::mt19937 g(seed);
  std::normal_distribution<double> nd(0.0, 1.0);
  std::uniform_int_distribution<int> ui(0, (int)S_kv - 1);
  std::vector<R> q(B * S * H * D), kv(B * S_kv * D), o(B * S * H * D), dout(B * S * H * D);
  for (auto& v : q) v = (R)nd(g);
  for (auto& v : kv) v = (R)nd(g);
  for (auto& v : dout) v = (R)nd(g);
  std::vector<float> sink(H);
  for (auto& v : sink) v = (float)nd(g);
  sink[0] = -std::numeric_limits<float>::infinity();
  std::vector<int32_t> idx(B * S * topk);
  const int32_t bad[4] = {-1, std::numeric_limits<int32_t>::min(), (int32_t)S_kv, std::numeric_limits<int32_t>::max()};
  for (int64_t k = 0; k < (int64_t)idx.size(); k++) idx[k] = (k % 7 == 3) ? bad[(k / 7) % 4] : ui(g);
  for (int64_t t = 0; t < topk; t++) idx[t] = -1;                  // token 0: fully masked
  if (topk > 1) idx[topk + 1] = idx[topk];                          // token 1: a row twice
  const double sm = 1.0 / std::sqrt((double)D);
  std::vector<R> lse(B * S * H), dq(B * S * H * D), delta(B * S * H), dkv(B * S_kv * D);
  run_fwd<R>(q.data(), kv.data(), sink.data(), idx.data(), B, S, S_kv, H, D, topk, sm, nullptr, 0, o.data(),
             lse.data());
  run_dq<R>(q.data(), kv.data(), o.data(), dout.data(), idx.data(), lse.data(), B, S, S_kv, H, D, topk, sm, nullptr,
            0, dq.data(), delta.data());
  run_dkv<R>(q.data(), kv.data(), o.data(), dout.data(), idx.data(), lse.data(), B, S, S_kv, H, D, topk, sm, nullptr,
             0, dkv.data());
  // explicit lists (the last token and row first, one entry twice)
  const int64_t toks[3] = {B * S - 1, 0, B * S - 1};
  const int64_t rows[3] = {B * S_kv - 1, 0, 1};
  std::vector<R> o2(3 * H * D), lse2(3 * H), dq2(3 * H * D), dkv2(3 * D);
  run_fwd<R>(q.data(), kv.data(), sink.data(), idx.data(), B, S, S_kv, H, D, topk, sm, toks, 3, o2.data(), lse2.data());
  run_dq<R>(q.data(), kv.data(), o.data(), dout.data(), idx.data(), lse.data(), B, S, S_kv, H, D, topk, sm, toks, 3,
            dq2.data(), nullptr);
  run_dkv<R>(q.data(), kv.data(), o.data(), dout.data(), idx.data(), lse.data(), B, S, S_kv, H, D, topk, sm, rows, 3,
             dkv2.data());
  int bad_count = 0;
  for (auto v : o) bad_count += !std::isfinite((double)v);
  for (auto v : dq) bad_count += !std::isfinite((double)v);
  for (auto v : dkv) bad_count += !std::isfinite((double)v);
  for (int64_t k = 0; k < B * S * H; k++) {  // LSE is -inf only for a fully masked token's sinkless head
    const int64_t token = k / H, b = token / S;
    bool any = false;
    for (int64_t t = 0; t < topk; t++) any |= in_range(idx[token * topk + t], S_kv);
    (void)b;
    bad_count += !std::isfinite((double)lse[k]) && (any || k % H != 0);
  }
  for (int64_t k = 0; k < 3 * H * D; k++) bad_count += o2[k] != o[toks[k / (H * D)] * H * D + k % (H * D)];
  for (int64_t k = 0; k < 3 * D; k++) bad_count += dkv2[k] != dkv[rows[k / D] * D + k % D];
  return bad_count;
}

}  // namespace

int main() {
  int bad = 0;
  bad += run_case<float>(2, 9, 23, 4, 16, 11, 1);
  bad += run_case<double>(2, 9, 23, 4, 16, 11, 2);
  bad += run_case<float>(1, 40, 64, 2, 32, 37, 3);
  bad += run_case<double>(3, 5, 7, 3, 8, 1, 4);
  std::printf("oracle sanitizer driver: %d unexpected values\n", bad);
  return bad == 0 ? 0 : 1;
}
