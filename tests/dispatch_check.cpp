// Host driver for tests/test_dispatch_host.py: reads "M N K cus" lines and
// prints the GEMM kernel the dispatch rules choose for each.
#include <stdio.h>

#include "../int8_w8a8_quantized_token_amd/csrc/gemm_dispatch.h"

int main() {
  long long M, N, K, cus;
  while (scanf("%lld %lld %lld %lld", &M, &N, &K, &cus) == 4) {
    using namespace w8a8::dispatch;
    if (mid_path(M, N, K)) {
      const MidConfig m = mid_config(M, N, K, cus);
      printf("mid %d %d %d %d\n", m.mt, m.rw, m.nw, m.ns);
    } else if (K % kMidBK == 0 && M > kSkinnyMaxM) {
      const PrefillTile t = prefill_tile(M, N, cus);
      printf("prefill %s\n", t == PrefillTile::k256x192 ? "256x192"
                             : t == PrefillTile::k192x256 ? "192x256" : "256x256");
    } else {
      printf("other\n");
    }
  }
  return 0;
}
