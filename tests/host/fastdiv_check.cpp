// Check of the kernels' magic-number division (FastDiv in csrc/launch.h):
// every divisor below 5000 against plain division on 20000 small numerators,
// random numerators below 2^31 and the largest one, then random divisors up
// to 2^31.  The device code computes (mulhi(n, m) + n) >> l exactly as here.
// Built and run by tests/test_capi_host.py.
#include "launch.h"
#include <cstdio>
#include <random>
using namespace rgg;
static uint32_t fdiv(uint32_t n, const FastDiv& f){ return (uint32_t)((((uint64_t)n * f.m) >> 32) + n) >> f.l; }
int main(){
  std::mt19937_64 r(1);
  for (uint32_t d=1; d<5000; ++d){ FastDiv f=make_fastdiv(d);
    for (uint32_t n=0;n<20000;++n) if (fdiv(n,f)!=n/d){printf("bad d=%u n=%u\n",d,n);return 1;}
    for (int k=0;k<2000;++k){ uint32_t n=r()%(1u<<31); if (fdiv(n,f)!=n/d){printf("bad d=%u n=%u\n",d,n);return 1;} }
    uint32_t n=(1u<<31)-1; if (fdiv(n,f)!=n/d){printf("bad max d=%u\n",d);return 1;}
  }
  for (int k=0;k<200000;++k){ uint32_t d=1+r()%(1u<<31); FastDiv f=make_fastdiv(d); uint32_t n=r()%(1u<<31); if (fdiv(n,f)!=n/d){printf("bad d=%u n=%u\n",d,n);return 1;} }
  printf("fastdiv ok\n");
}
