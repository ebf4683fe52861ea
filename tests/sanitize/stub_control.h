// stub_control.h -- controls of the host-memory HIP stand-in (hip_stub.cpp).
#pragma once
#ifdef __cplusplus
extern "C" {
#endif
void stub_fail_malloc_at(int k);   // the k-th hipMalloc from now fails (-1: none)
long stub_live_allocations(void);  // hipMalloc'd blocks not yet freed
long stub_launches(void);          // launcher calls that passed their checks
void stub_set_num_cu(int n);       // compute units the stand-in device reports
#ifdef __cplusplus
}
#endif
