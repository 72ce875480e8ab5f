// Driver of the host-only sanitizer build of the planner.  Reads requests
// from the file named by argv[1], each laid out as the C ABI's own structs:
//   int32 n_tensors, int32 n_preconds,
//   n_tensors x muon_tensor_t, n_preconds x muon_precond_t, muon_hparams_t
// and for each prints the status and workspace bytes of muon_workspace_size
// and, when that succeeds, the JSON of muon_plan_describe (or the error
// text).  The descriptors are copied into arrays of exactly their length, so
// an out-of-bounds read of them is caught by AddressSanitizer.  No GPU call.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "muon.h"

template <typename T>
static bool read_n(FILE* f, std::vector<T>& v, size_t n) {
  v.resize(n);
  return n == 0 || std::fread(v.data(), sizeof(T), n, f) == n;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s requests.bin\n", argv[0]);
    return 2;
  }
  FILE* f = std::fopen(argv[1], "rb");
  if (!f) {
    std::perror(argv[1]);
    return 2;
  }
  for (int k = 0;; ++k) {
    int32_t counts[2];
    if (std::fread(counts, sizeof(int32_t), 2, f) != 2) break;
    std::vector<muon_tensor_t> ts;
    std::vector<muon_precond_t> pcs;
    std::vector<muon_hparams_t> hp;
    if (counts[0] < 0 || counts[1] < 0 || !read_n(f, ts, size_t(counts[0])) ||
        !read_n(f, pcs, size_t(counts[1])) || !read_n(f, hp, 1)) {
      std::fprintf(stderr, "request %d: truncated\n", k);
      return 2;
    }
    const muon_tensor_t* tp = ts.empty() ? nullptr : ts.data();
    const muon_precond_t* pp = pcs.empty() ? nullptr : pcs.data();
    size_t bytes = 0;
    muon_status_t st = muon_workspace_size(tp, counts[0], pp, counts[1], hp.data(), &bytes);
    std::printf("request %d status %s bytes %zu\n", k, muon_status_str(st), bytes);
    if (st != MUON_OK) {
      std::printf("error %s\n", muon_last_error());
      continue;
    }
    size_t need = 0;
    st = muon_plan_describe(tp, counts[0], pp, counts[1], hp.data(), nullptr, 0, &need);
    std::vector<char> buf(need + 1, 0);
    if (st == MUON_OK) st = muon_plan_describe(tp, counts[0], pp, counts[1], hp.data(), buf.data(), buf.size(), &need);
    if (st != MUON_OK) {
      std::printf("plan-error %s %s\n", muon_status_str(st), muon_last_error());
      continue;
    }
    std::printf("plan %s\n", buf.data());
  }
  std::fclose(f);
  return 0;
}
