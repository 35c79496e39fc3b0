"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path."""
from .gen import (DTYPES, ELEM_BYTES, MQ_WORKLOADS, WORKLOADS, Case, MQCase, assign_blocks,
                  encode, gather_logical, layout_cache, make_case, make_mq_case, mq_workload,
                  poison_fill, workload, workload_lengths)

__all__ = ["DTYPES", "ELEM_BYTES", "MQ_WORKLOADS", "WORKLOADS", "Case", "MQCase",
           "assign_blocks", "encode", "gather_logical", "layout_cache", "make_case",
           "make_mq_case", "mq_workload", "poison_fill", "workload", "workload_lengths"]
